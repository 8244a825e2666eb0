// jb_prefill.hip -- chunked gated delta-rule prefill for gfx950.
//
// The recurrence (JetBlock time mixing is Gated DeltaNet: Jet-Nemotron csdn
// translation, section 2.4) in the transposed state M = S^T (dk x dv):
//     M_t = a_t (I - b_t k_t k_t^T) M_{t-1} + b_t k_t v'_t^T,   o_t = M_t^T q_t
// with L2-normalised q, k.  Within a chunk of C = 64 tokens entering with M0
// (local index i, g_i = sum_{j<=i} ln a_j, gamma_i = e^{g_i}):
//     A_ij = b_i e^{g_i - g_j} k_i.k_j (j < i)
//     W = (I + A)^{-1} diag(b gamma) K,  U0 = (I + A)^{-1} diag(b) V'   (WY/UT form)
//     V_new = U0 - W M0
//     O = diag(gamma) Q M0 + P V_new,  P_ij = e^{g_i - g_j} q_i.k_j (j <= i)
//     M_C = gamma_C M0 + K^T diag(e^{g_C - g}) V_new
// so a chunk maps M0 to Phi_c M0 + D_c.  A long sequence is cut into
// segments of L chunks; three kernels then run:
//   1. summary  (per segment but the last, in parallel): the segment's affine
//      map (Phi_s, D_s), obtained by running the chunk loop from the zero
//      state on the augmented columns [D | Phi] with Phi starting at I;
//   2. scan     (per head and 16-column tile): M_{s+1} = Phi_s M_s + D_s;
//   3. output   (per segment, in parallel): the chunk loop from the true M_s,
//      writing o and, for the last segment, the final state.
// With one segment only the output kernel runs.
//
// Matrix products run on the matrix cores: fp16 operands with fp32
// accumulation for bfloat16 inputs (bf16 inputs convert to fp16 exactly in
// the normal range), fp32 operands in the all-fp32 mode.  The state and every
// accumulator stay fp32; scalars (norms, gates) are applied in fp32.
//
// Workgroup: 8 wavefronts.  Chunk-shared tiles (K, K^T, Q, -A, the diagonal
// blocks of A and their inverses, -W, P, the value rows with their 3-row conv
// halo) live in LDS; each wave owns whole 16-column tiles of the state and
// keeps them in accumulator registers for the whole segment, so the state
// never leaves the compute unit.  (I + A)^{-1} is never formed: only its four
// 16x16 diagonal blocks are inverted (fp32, forward substitution), and every
// wave applies a blocked forward substitution on the matrix cores to its own
// right-hand sides (its columns of diag(b) V', and one column tile of
// diag(b gamma) K for the W tiles).
#include <algorithm>

#include "jb_chunk.h"
#include "jb_device.h"
#include "jb_internal.h"

namespace jb {

// MODE_CKPT runs the output pass's state recurrence without q, P and o and
// stores the state entering every chunk (the backward pass starts from them).
enum { MODE_SUMMARY = 0, MODE_OUTPUT = 1, MODE_CKPT = 2 };

// the chunk kernel also forms Q^T-side tiles (normalised q, P) in output mode
__host__ __device__ constexpr bool with_q(int mode) { return mode == MODE_OUTPUT; }

struct ChunkArgs {
  int T, H, nchunks, seg_len, nseg;
  // packed sequences of different lengths: sequence b is rows cu_seqlens[b] ..
  // cu_seqlens[b+1] - 1 of the token-major tensors, at most T of them (NULL:
  // every sequence has T tokens, rows b T .. b T + T - 1)
  const int* cu_seqlens;
  int64_t total;        // rows of the token-major tensors (packed batches: cu_seqlens[B])
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* taps;
  const void* conv_in;
  // static-conv mode: fixed per-channel weights [H*d][4] and the q / k caches
  const float* wq;
  const float* wk;
  const float* wv;
  const void* cq_in;
  const void* ck_in;
  const float* S0;      // output kernel with one segment only
  const float* Mstart;  // [B][H][nseg][DK][DV] start states (several segments)
  float* Dsum;          // [B][H][nseg][DK][DV]
  float* Phi;           // [B][H][nseg][DK][DK]
  void* o;
  float* S_final;
  _Float16* Mck;        // MODE_CKPT: the state entering every chunk, fp16 16x16 tiles (below)
  char* img;            // MODE_CKPT: per chunk, the K, -W^T and gate parts of ChainImg
  const float* ck_scale;  // MODE_CKPT: the stored states are the true states times *ck_scale (a power of two)
};

// ------------------------------------------------------------ LDS layout
//
// Every tile row is padded by 4 elements: a fragment read has the 16 lanes of
// a lane group walk 16 rows at one column, and an unpadded 128- or 192-byte
// row stride would put all of them in one or two LDS banks.  With the pad the
// row stride is 2 (mod 4) dwords for fp16 and 4 (mod 8) dwords for fp32
// tiles, so the lanes of a group spread over distinct banks.

template <int DK, int DV, typename IO, typename OP, int MODE, bool SC>
struct Lds {
  static constexpr int LDK = DK + 4;                     // [C][DK] tiles
  static constexpr int LC = C + 4;                       // [*][C] tiles
  static constexpr int LVB = DV * (int)sizeof(IO);       // bytes per value row (DMA-filled, unpadded)
  static constexpr int LAD = 16 + 4;                     // fp32 diagonal blocks of A
  static constexpr int LLI = 32 + 4;                     // diagonal-block inverses (cols 16..31 zero)
  static constexpr int szKh = C * LDK * (int)sizeof(OP);
  static constexpr int szKt = DK * LC * (int)sizeof(OP);
  static constexpr int szQh = with_q(MODE) ? C * LDK * (int)sizeof(OP) : 0;
  static constexpr int szV = (C + 3) * LVB;
  static constexpr int szTap = SC ? 0 : C * 4 * 4;
  static constexpr int szScal = 4 * C * 4;
  static constexpr int szW = C * LDK * (int)sizeof(OP);
  static constexpr int szAn = C * LC * (int)sizeof(OP);
  static constexpr int szAd = C * LAD * 4;
  static constexpr int szLi = C * LLI * (int)sizeof(OP);
  static constexpr int szP = with_q(MODE) ? C * LC * (int)sizeof(OP) : 0;
  // raw q or k rows of a chunk (static conv: with the 3-row halo in front, like the values)
  static constexpr int szRaw = (SC ? C + 3 : C) * DK * (int)sizeof(IO);
  static constexpr int szQraw = with_q(MODE) ? szRaw : 0;
  static constexpr int szGraw = C * 4 * 2 + (SC ? 0 : C * 16);             // raw alpha, beta, taps
  // bf16 inputs: the band T of the right-hand side diag(b) V' = T V_ext, as
  // [hi, lo][row tile][16 rows][LT] bf16 (32 columns used)
  static constexpr int LT = 32 + 8;
  static constexpr int szT = sizeof(IO) == 2 && !SC ? 2 * 4 * 16 * LT * 2 : 0;
  // static conv: the head's weights, q and k tap-major [4][DK] f32 each, v as one float4 per column [DV]
  static constexpr int szCw = SC ? (2 * DK + DV) * 16 : 0;

  static constexpr int a16(int x) { return (x + 15) / 16 * 16; }
  // small per-row arrays first, then the raw q / k staging (the -A region
  // doubles as raw k staging) and the tiles read with the C-element row
  // stride: a ds_read immediate offset reaches 64 KB, so everything placed
  // below that is addressed from one lane-dependent register per row stride
  static constexpr int oGraw = 0;
  static constexpr int oTap = a16(oGraw + szGraw);
  static constexpr int oScal = a16(oTap + szTap);
  static constexpr int oQraw = a16(oScal + szScal);
  static constexpr int oAn = a16(oQraw + szQraw);
  static constexpr int oAd = a16(oAn + szAn);
  static constexpr int oLi = a16(oAd + szAd);
  static constexpr int oKt = a16(oLi + szLi);
  static constexpr int oP = a16(oKt + szKt);
  static constexpr int oW = a16(oP + szP);
  static constexpr int oQh = a16(oW + szW);
  static constexpr int oKh = a16(oQh + szQh);
  static constexpr int oV = a16(oKh + szKh);
  static constexpr int oT = a16(oV + szV);
  static constexpr int oCw = a16(oT + szT);
  static constexpr int total = a16(oCw + szCw);
  // raw k rows of the next chunk land in the -A / diagonal-block region, dead
  // while a chunk's column phase runs and rewritten only after the prologue
  static constexpr int oKraw = oAn;
  static_assert(oLi + szLi - oAn >= szRaw, "raw k staging does not fit");
};

// ------------------------------------------------------------ chunk kernel


template <int DK, int DV, typename IO, typename OP, typename OUT, int MODE, bool SC>
__global__ __launch_bounds__(NTHR, 1) void chunk_kernel(ChunkArgs a) {
  using L = Lds<DK, DV, IO, OP, MODE, SC>;
  constexpr int LDK = L::LDK, LC = L::LC, LVB = L::LVB, LAD = L::LAD, LLI = L::LLI;
  constexpr int NCT = MODE == MODE_SUMMARY ? (DV + DK) / 16 : DV / 16;  // column tiles
  constexpr int CPW = (NCT + NWAVE - 1) / NWAVE;                        // tiles per wave (max)
  constexpr int RT = DK / 16;                                           // row tiles of M
  constexpr int KB = DK / 32;                                           // 32-deep blocks of dk
  constexpr int VCT = DV / 16;                                          // value column tiles
  static_assert(L::total <= 160 * 1024, "LDS budget of one CU exceeded");
  static_assert(RT <= NWAVE, "one wave per W column tile");

  __shared__ __attribute__((aligned(16))) char smem[L::total];
  OP* sKh = reinterpret_cast<OP*>(smem + L::oKh);           // [C][LDK]  normalised k
  OP* sKt = reinterpret_cast<OP*>(smem + L::oKt);           // [DK][LC]  its transpose
  OP* sQh = reinterpret_cast<OP*>(smem + L::oQh);           // [C][LDK]  normalised q
  char* sV = smem + L::oV;                                  // [C+3] rows of LVB bytes: raw v, t0-3 ..
  float* sTap = reinterpret_cast<float*>(smem + L::oTap);   // [C][4]
  float* sG = reinterpret_cast<float*>(smem + L::oScal);    // [C] g / ln 2
  float* sGam = sG + C;                                     // [C] e^g
  float* sBeta = sG + 2 * C;                                // [C] b
  float* sDec = sG + 3 * C;                                 // [C] e^{g_C - g}
  OP* sW = reinterpret_cast<OP*>(smem + L::oW);             // [C][LDK]  -W
  OP* sAn = reinterpret_cast<OP*>(smem + L::oAn);           // [C][LC]   -A (lower tiles)
  float* sAd = reinterpret_cast<float*>(smem + L::oAd);     // [C][LAD]  diagonal blocks of A
  OP* sLi = reinterpret_cast<OP*>(smem + L::oLi);           // [C][LLI]  their inverses
  OP* sP = reinterpret_cast<OP*>(smem + L::oP);             // [C][LC]   gated causal Q K^T
  char* sKraw = smem + L::oKraw;                            // [C][DK] raw k of the next chunk
  char* sQraw = smem + L::oQraw;                            // [C][DK] raw q of the next chunk
  char* sGraw = smem + L::oGraw;                            // raw alpha [C], beta [C], taps [C][4]
  bf16_t* sT = reinterpret_cast<bf16_t*>(smem + L::oT);     // bf16 inputs: band T, hi then lo
  float* sCwq = reinterpret_cast<float*>(smem + L::oCw);    // static conv weights: q [4][DK], k [4][DK],
  float* sCwk = sCwq + 4 * DK;                              // v [DV] float4
  const float4* sCwv = reinterpret_cast<const float4*>(sCwk + 4 * DK);

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = a.H;
  int64_t tok0;
  int T;
  seq_span(a.cu_seqlens, a.T, a.total, b, tok0, T);
  const int nseg_b = seq_segments(T, a.seg_len);
  // a packed batch plans its grid for the longest sequence: shorter ones
  // leave the extra segments' workgroups idle (the summary kernel has one
  // workgroup per segment but the last)
  if (s >= (MODE == MODE_SUMMARY ? nseg_b - 1 : nseg_b)) return;
  // the wave index is uniform across a wave: keep it (and what derives from it) in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int m16 = lane & 15, g4 = lane >> 4;
  const IO* q = reinterpret_cast<const IO*>(a.q);
  const IO* k = reinterpret_cast<const IO*>(a.k);
  const IO* v = reinterpret_cast<const IO*>(a.v);
  const IO* cin = reinterpret_cast<const IO*>(a.conv_in);
  const int64_t bh = (int64_t)b * H + h;

  // ---- initial state (accumulator layout: lane holds M[rt*16+4g+i][ct*16+m16])
  f4_t Macc[CPW][RT];
  // fp16 operands: each column tile held at its own power-of-two scale (jb_chunk.h)
  constexpr bool SCALED = sizeof(OP) == 2;
  int Ex[CPW];
#pragma unroll
  for (int cw = 0; cw < CPW; ++cw) Ex[cw] = E_FRESH;
#pragma unroll
  for (int cw = 0; cw < CPW; ++cw) {
    const int ct = wave + cw * NWAVE;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      Macc[cw][rt] = zero4();
      if (ct >= NCT) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + 4 * g4 + i;
        if (MODE == MODE_SUMMARY) {
          if (ct >= VCT) Macc[cw][rt][i] = (row == (ct - VCT) * 16 + m16) ? 1.f : 0.f;
        } else {
          const int col = ct * 16 + m16;
          const float* src = a.nseg > 1 ? a.Mstart + ((bh * a.nseg + s) * DK) * DV
                                        : (a.S0 ? a.S0 + bh * DK * DV : nullptr);
          Macc[cw][rt][i] = src ? src[row * DV + col] : 0.f;
        }
      }
    }
  }

  // P above its block diagonal is never written by the chunk loop
  if (with_q(MODE))
    for (int e = tid; e < C * C; e += NTHR) {
      const int r = e / C, c = e % C;
      if ((c >> 4) > (r >> 4)) sP[r * LC + c] = from_f32<OP>(0.f);
    }
  // static conv: the head's weights stay in LDS for the whole segment
  if constexpr (SC)
    for (int e = tid; e < 2 * DK + DV; e += NTHR) {
      if (e < 2 * DK) {
        const int d = e % DK;
        const float4 w = *reinterpret_cast<const float4*>((e < DK ? a.wq : a.wk) + ((int64_t)h * DK + d) * 4);
        float* dst = e < DK ? sCwq : sCwk;
        dst[d] = w.x;
        dst[DK + d] = w.y;
        dst[2 * DK + d] = w.z;
        dst[3 * DK + d] = w.w;
      } else {
        const_cast<float4*>(sCwv)[e - 2 * DK] =
            *reinterpret_cast<const float4*>(a.wv + ((int64_t)h * DV + e - 2 * DK) * 4);
      }
    }

  const int c_begin = s * a.seg_len;
  const int c_end = min((T + C - 1) / C, c_begin + a.seg_len);

  // Raw inputs of chunk cc straight into LDS: value rows t0-3 .. t0+63 into
  // sV (zeros where neither v nor the conv cache has a row), raw k (and q)
  // rows into their staging tiles, and the gates.  Rows at or beyond the
  // sequence end are skipped; the prologue treats them as neutral tokens.
  auto issue_chunk = [&](int cc) {
    const int t0c = cc * C, nc = min(C, T - t0c);
    constexpr int EP = 16 / (int)sizeof(IO);            // elements per 16-byte piece
    constexpr int PPR = DV / EP;                        // pieces per value row
    constexpr int NPV = (C + 3) * PPR;
    for (int j = wave; j * 64 < NPV; j += NWAVE) {
      const int p = j * 64 + lane;
      if (p < NPV) {
        const int r = p / PPR, pc = p % PPR, t = t0c - 3 + r;
        if (t >= 0 && r - 3 < nc)
          dma16(v + ((tok0 + t) * H + h) * DV + pc * EP, sV + j * 64 * 16);
        else if (t < 0 && cin)
          dma16(cin + (((int64_t)b * 3 + (3 + t)) * H + h) * DV + pc * EP, sV + j * 64 * 16);
        else
          *reinterpret_cast<uint4*>(sV + p * 16) = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    constexpr int PPK = DK / EP;                        // pieces per q or k row
    if constexpr (!SC) {
      for (int j = wave; j * 64 < C * PPK; j += NWAVE) {
        const int p = j * 64 + lane;
        const int r = p / PPK, pc = p % PPK;
        if (p < C * PPK && r < nc) {
          const int64_t off = ((tok0 + t0c + r) * H + h) * DK + pc * EP;
          dma16(k + off, sKraw + j * 64 * 16);
          if (with_q(MODE)) dma16(q + off, sQraw + j * 64 * 16);
        }
      }
    } else {
      // static conv: q and k rows t0-3 .. t0+63 like the values; rows past
      // the sequence end are left as they are (the prologue never reads them)
      const IO* cq = reinterpret_cast<const IO*>(a.cq_in);
      const IO* ck = reinterpret_cast<const IO*>(a.ck_in);
      constexpr int NPK = (C + 3) * PPK;
      for (int j = wave; j * 64 < NPK; j += NWAVE) {
        const int p = j * 64 + lane;
        if (p < NPK) {
          const int r = p / PPK, pc = p % PPK, t = t0c - 3 + r;
          if (t >= 0) {
            if (r - 3 < nc) {
              const int64_t off = ((tok0 + t) * H + h) * DK + pc * EP;
              dma16(k + off, sKraw + j * 64 * 16);
              if (with_q(MODE)) dma16(q + off, sQraw + j * 64 * 16);
            }
          } else if (ck) {
            const int64_t off = (((int64_t)b * 3 + (3 + t)) * H + h) * DK + pc * EP;
            dma16(ck + off, sKraw + j * 64 * 16);
            if (with_q(MODE)) dma16(cq + off, sQraw + j * 64 * 16);
          } else {
            *reinterpret_cast<uint4*>(sKraw + p * 16) = make_uint4(0u, 0u, 0u, 0u);
            if (with_q(MODE)) *reinterpret_cast<uint4*>(sQraw + p * 16) = make_uint4(0u, 0u, 0u, 0u);
          }
        }
      }
    }
    if (wave == GATE_WAVE && lane < nc) {
      const int64_t gidx = (tok0 + t0c + lane) * H + h;
      dma4(a.alpha + gidx, sGraw);
      dma4(a.beta + gidx, sGraw + C * 4);
      if constexpr (!SC) dma16(a.taps + gidx * 4, sGraw + C * 8);
    }
  };

  // a column tile of outputs, rows t0 .. t0+n-1, straight from registers
  auto store_o = [&](const f4_t (&Ot)[4], int ct, int t0, int n, int E) {
    const uint32_t rowb = (uint32_t)(H * DV * (int)sizeof(OUT));
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(reinterpret_cast<OUT*>(a.o) + ((tok0 + t0) * H + h) * DV, (uint32_t)n * rowb);
    const int ovoff = (int)(4 * g4 * rowb) + (ct * 16 + m16) * (int)sizeof(OUT);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        // rows at or beyond n fall outside the resource and are dropped
        buf_store(orsrc, from_f32<OUT>(SCALED ? ldexpf(Ot[rt][i], held_exp(E)) : Ot[rt][i]), ovoff,
                  (int)((rt * 16 + i) * rowb));
  };

  // T is zero outside its band; the band is rewritten every chunk
  for (int e = tid; e < L::szT / 16; e += NTHR) reinterpret_cast<uint4*>(smem + L::oT)[e] = make_uint4(0u, 0u, 0u, 0u);
  if (c_begin < c_end) issue_chunk(c_begin);

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * C;
    const int n = min(C, T - t0);
    if constexpr (MODE == MODE_CKPT) {
      // the state entering chunk c, for the backward pass, in the fp16 its
      // products there take as an operand and in accumulator tiles: per chunk
      // [DV/16][DK/16][64 lanes][4], lane l of tile (ct, rt) holding rows
      // 16 rt + 4 (l / 16) .. + 3 of column 16 ct + l % 16 (one 8-byte store)
      _Float16* dst = a.Mck + ((bh * a.nchunks + c) * DK) * DV;
      const float cks = a.ck_scale ? *a.ck_scale : 1.f;
#pragma unroll
      for (int cw = 0; cw < CPW; ++cw) {
        const int ct = wave + cw * NWAVE;
        if (ct < NCT)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int ce = held_exp(Ex[cw]);
            const half4_t hv = {(_Float16)(ldexpf(Macc[cw][rt][0], ce) * cks),
                                (_Float16)(ldexpf(Macc[cw][rt][1], ce) * cks),
                                (_Float16)(ldexpf(Macc[cw][rt][2], ce) * cks),
                                (_Float16)(ldexpf(Macc[cw][rt][3], ce) * cks)};
            *reinterpret_cast<half4_t*>(dst + ((ct * RT + rt) * 64 + lane) * 4) = hv;
          }
      }
    }

    // ================= prefetched inputs -> prologue =================
    __builtin_amdgcn_s_waitcnt(0);  // this wave's LDS DMA transfers have landed
    __syncthreads();                // ... and every other wave's
    {
      if (SC && tid < PRO_THR) {
        // static conv: thread (row, part) as in Prologue; the convolved rows
        // are formed twice, once for their norms and once to be scaled and
        // stored, so that no thread holds a whole row part at a time
        constexpr int E = DK / 8;
        const int row = tid >> 3, d0 = (tid & 7) * E;
        const bool valid = row < n;
        const IO* kraw = reinterpret_cast<const IO*>(sKraw);
        const IO* qraw = reinterpret_cast<const IO*>(sQraw);
        float sk = 0.f, sq = 0.f;
        // rolled loops: unrolled, the addresses of every group would be
        // hoisted out of the chunk loop and spilled
#pragma unroll 1
        for (int e0 = 0; e0 < E; e0 += 4) {
          const int dd = d0 + e0;
          float x[4];
          conv4<DK, IO>(kraw, sCwk, row, dd, valid, x);
#pragma unroll
          for (int i = 0; i < 4; ++i) sk += x[i] * x[i];
          if (with_q(MODE)) {
            conv4<DK, IO>(qraw, sCwq, row, dd, valid, x);
#pragma unroll
            for (int i = 0; i < 4; ++i) sq += x[i] * x[i];
          }
        }
        const float rk = l2_scale(group_sum<8>(sk));
        const float rq = with_q(MODE) ? l2_scale(group_sum<8>(sq)) : 0.f;
#pragma unroll 1
        for (int e0 = 0; e0 < E; e0 += 4) {
          const int dd = d0 + e0;
          float x[4];
          conv4<DK, IO>(kraw, sCwk, row, dd, valid, x);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const OP kh = from_f32<OP>(x[i] * rk);
            sKh[row * LDK + dd + i] = kh;
            sKt[(dd + i) * LC + row] = kh;
          }
          if (with_q(MODE)) {
            conv4<DK, IO>(qraw, sCwq, row, dd, valid, x);
#pragma unroll
            for (int i = 0; i < 4; ++i) sQh[row * LDK + dd + i] = from_f32<OP>(x[i] * rq);
          }
        }
      } else if (tid < PRO_THR) {
        Prologue<DK, IO> pr;
        pr.load(reinterpret_cast<const IO*>(sQraw), reinterpret_cast<const IO*>(sKraw), 0, 1, n,
                with_q(MODE));
        pr.finish(with_q(MODE));
#pragma unroll
        for (int e = 0; e < Prologue<DK, IO>::E; ++e) {
          const int d = pr.part * Prologue<DK, IO>::E + e;
          const OP kh = from_f32<OP>(pr.kv[e]);
          sKh[pr.row * LDK + d] = kh;
          sKt[d * LC + pr.row] = kh;
          if (with_q(MODE)) sQh[pr.row * LDK + d] = from_f32<OP>(pr.qv[e]);
        }
      }
      if (wave == GATE_WAVE) {
        const bool valid = lane < n;
        const float al = valid ? reinterpret_cast<const float*>(sGraw)[lane] : 1.f;
        const float be = valid ? reinterpret_cast<const float*>(sGraw + C * 4)[lane] : 0.f;
        const float4 tp = valid && !SC ? reinterpret_cast<const float4*>(sGraw + C * 8)[lane]
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
        const float g = chunk_gate_scan(al);
        const float gC = __shfl(g, C - 1, WAVE);
        sG[lane] = g;
        sGam[lane] = fast_exp2(g);
        sBeta[lane] = be;
        sDec[lane] = fast_exp2(gC - g);
        if constexpr (!SC) *reinterpret_cast<float4*>(sTap + lane * 4) = tp;
        if constexpr (sizeof(IO) == 2 && !SC) {
          // row `lane` of the band T with T[r][r + j] = b_r tap_r[j], so that the
          // right-hand side diag(b) V' = T V_ext runs on the matrix cores; row
          // tile rt multiplies the 32 staged value rows from 16 rt (from 35 for
          // the last tile, which keeps the window inside the C + 3 rows), and
          // each coefficient is split into bf16 hi + lo
          const int rt = lane >> 4, m = lane & 15, k0 = (rt < 3 ? 0 : 16 * rt - (C + 3 - 32)) + m;
          const float cf[4] = {be * tp.x, be * tp.y, be * tp.z, be * tp.w};
          bf16_t* th = sT + (rt * 16 + m) * L::LT + k0;
          bf16_t* tl = th + 4 * 16 * L::LT;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16_t hi = f32_to_bf16(cf[j]);
            th[j] = hi;
            tl[j] = f32_to_bf16(cf[j] - bf16_to_f32(hi));
          }
        }
      }
    }
    __syncthreads();

    f4_t U[CPW][4];
    // ================= K K^T -> -A (and its diagonal blocks), Q K^T -> P =================
    {
      constexpr int NJOB = with_q(MODE) ? 20 : 10;
      for (int job = wave; job < NJOB; job += NWAVE) {
        const int which = job >= 10, t = job - 10 * which;
        const int ti = (kLowI >> (2 * t)) & 3, tj = (kLowJ >> (2 * t)) & 3;
        const OP* Asrc = which ? sQh : sKh;
        f4_t acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          mma(acc, lds_frag<OP>(Asrc, LDK, ti * 16, kb * 32), lds_frag<OP>(sKh, LDK, tj * 16, kb * 32));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = ti * 16 + 4 * g4 + i, cc = tj * 16 + m16;
          if (which == 0) {
            const float av = cc < r ? sBeta[r] * fast_exp2(sG[r] - sG[cc]) * acc[i] : 0.f;
            sAn[r * LC + cc] = from_f32<OP>(-av);
            if (ti == tj) sAd[r * LAD + m16] = av;
          } else {
            sP[r * LC + cc] = from_f32<OP>(cc <= r ? fast_exp2(sG[r] - sG[cc]) * acc[i] : 0.f);
          }
        }
      }
    }
    __syncthreads();


    // ================= diagonal-block inverses (wave 0) =================
    if (wave == 0) {
      // four 16x16 blocks by forward substitution, one column per lane; rows
      // are read as float4 and the scheduling fences keep the compiler from
      // hoisting all 120 row values into registers at once
      const int base = (lane >> 4) * 16, jc = lane & 15;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == jc) ? 1.f : 0.f;
        const float* arow = sAd + (base + i) * LAD;
#pragma unroll
        for (int k4 = 0; k4 < i; k4 += 4) {
          const float4 av = *reinterpret_cast<const float4*>(arow + k4);
          acc -= av.x * x[k4];
          if (k4 + 1 < i) acc -= av.y * x[k4 + 1];
          if (k4 + 2 < i) acc -= av.z * x[k4 + 2];
          if (k4 + 3 < i) acc -= av.w * x[k4 + 3];
        }
        x[i] = acc;
        if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sLi[(base + i) * LLI + jc] = from_f32<OP>(x[i]);
        sLi[(base + i) * LLI + 16 + jc] = from_f32<OP>(0.f);  // the zero half a 32-deep fragment reads
      }
    }
    __syncthreads();

    // ================= per-wave solves: W tiles and U0 = (I+A)^{-1} diag(b) V' =================
    if (wave < RT) {
      // W = (I+A)^{-1} diag(b gamma) K, column tile `wave`; stored negated
      f4_t Y[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rb * 16 + 4 * g4 + i;
          Y[rb][i] = sBeta[r] * sGam[r] * to_f32<OP>(sKh[r * LDK + wave * 16 + m16]);
        }
      block_solve<OP, LC, LLI>(Y, sAn, sLi);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sW[(rb * 16 + 4 * g4 + i) * LDK + wave * 16 + m16] = from_f32<OP>(-Y[rb][i]);
    }
#pragma unroll
    for (int cw = 0; cw < CPW; ++cw) {
      const int ct = wave + cw * NWAVE;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) U[cw][rb] = zero4();
      if (ct >= NCT) continue;
      if (!(MODE == MODE_OUTPUT || ct < VCT)) {
        // a transition column (summary): no values, but its scale follows M
        if constexpr (SCALED) rescale_tile(Macc[cw], U[cw], Ex[cw]);
        continue;
      }
      // right-hand side diag(b) V', V'[r][col] = sum_j tap[r][j] v[t0 + r - 3 + j][col]
      const int col = ct * 16 + m16;
      if constexpr (SC) {
        // static conv, per-column weights: V'[r][col] = sum_j w[col].j v[t0 + r - 3 + j][col],
        // staged rows r .. r+3; the four rows of a lane share seven staged values
        int wc = col;
        asm volatile("" : "+v"(wc));  // read per chunk, not held across the loop
        const float4 w = sCwv[wc];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          float vr[7];
#pragma unroll
          for (int m = 0; m < 7; ++m)
            vr[m] = to_f32<IO>(reinterpret_cast<const IO*>(sV + (rb * 16 + 4 * g4 + m) * LVB)[col]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            U[cw][rb][i] = sBeta[rb * 16 + 4 * g4 + i] *
                           (w.x * vr[i] + w.y * vr[i + 1] + w.z * vr[i + 2] + w.w * vr[i + 3]);
        }
      } else if constexpr (sizeof(IO) == 2) {
        // on the matrix cores: U0 tile rt = (T_hi + T_lo) V_ext[window rows][this column tile],
        // the value rows taken exactly as bf16 operands (K order 8g + j on both sides)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int s0 = rt < 3 ? 16 * rt : C + 3 - 32;
          const bf16_t* vcol = reinterpret_cast<const bf16_t*>(sV + (s0 + 8 * g4) * L::LVB) + col;
          bf16x8_t vb;
#pragma unroll
          for (int j = 0; j < 8; ++j) vb[j] = __builtin_bit_cast(__bf16, vcol[j * (L::LVB / 2)]);
          const bf16x8_t th = *reinterpret_cast<const bf16x8_t*>(sT + (rt * 16 + m16) * L::LT + 8 * g4);
          const bf16x8_t tl = *reinterpret_cast<const bf16x8_t*>(sT + ((4 + rt) * 16 + m16) * L::LT + 8 * g4);
          const f4_t hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th, vb, zero4(), 0, 0, 0);
          U[cw][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl, vb, hi, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = rb * 16 + 4 * g4 + i;
            const float4 tp = *reinterpret_cast<const float4*>(sTap + r * 4);
            const IO* vcol = reinterpret_cast<const IO*>(sV + r * LVB) + col;
            const float vv = tp.x * to_f32<IO>(vcol[0]) + tp.y * to_f32<IO>(vcol[LVB / sizeof(IO)]) +
                             tp.z * to_f32<IO>(vcol[2 * LVB / sizeof(IO)]) + tp.w * to_f32<IO>(vcol[3 * LVB / sizeof(IO)]);
            U[cw][rb][i] = sBeta[r] * vv;
            if (i == 3) __builtin_amdgcn_sched_barrier(0);
          }
      }
      if constexpr (SCALED) rescale_tile(Macc[cw], U[cw], Ex[cw]);
      block_solve<OP, LC, LLI>(U[cw], sAn, sLi);
    }
    __syncthreads();

    // ================= state-dependent part, per column tile =================
    // the value rows, -A, its diagonal blocks and inverses, and the taps are
    // dead from here on: the next chunk's raw inputs can stream in now
    if (c + 1 < c_end) issue_chunk(c + 1);
    if constexpr (MODE == MODE_CKPT) {
      // the backward chain's K, -W^T and gate tiles of this chunk
      using I = ChainImg<DK>;
      char* im = a.img + (bh * a.nchunks + c) * I::bytes;
      for (int e = tid; e < C * (DK / 4); e += NTHR) {  // K rows, 8 bytes at a time
        const int r = e / (DK / 4), p = e % (DK / 4);
        *reinterpret_cast<uint2*>(im + I::oKh + (r * I::LK + p * 4) * 2) =
            *reinterpret_cast<const uint2*>(sKh + r * LDK + p * 4);
      }
      for (int e = tid; e < DK * (C / 2); e += NTHR) {  // -W^T, two rows of -W per 4-byte store
        const int d = e / (C / 2), r = (e % (C / 2)) * 2;
        const OP w0 = sW[r * LDK + d], w1 = sW[(r + 1) * LDK + d];
        *reinterpret_cast<uint32_t*>(im + I::oWt + (d * I::LT + r) * 2) =
            (uint32_t)__builtin_bit_cast(uint16_t, w0) | ((uint32_t)__builtin_bit_cast(uint16_t, w1) << 16);
      }
      if (tid < C) {
        reinterpret_cast<float*>(im + I::oGam)[tid] = sGam[tid];
        reinterpret_cast<float*>(im + I::oDec)[tid] = sDec[tid];
        reinterpret_cast<float*>(im + I::oG)[tid] = sG[tid];
      }
    }
    const float gamC = sGam[C - 1];
    if constexpr (CPW == 1) {
      // one column tile per wave
#pragma unroll
      for (int cw = 0; cw < CPW; ++cw) {
        const int ct = wave + cw * NWAVE;
        if (ct >= NCT) continue;
        // V_new = U0 - W M0 and (outputs) Q M0, sharing each M0 fragment
        f4_t O[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) O[rt] = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const Frag<OP> mf = acc_frag<OP>(Macc[cw][2 * kb], Macc[cw][2 * kb + 1]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) mma(U[cw][rt], lds_frag<OP>(sW, LDK, rt * 16, kb * 32), mf);
          if (MODE == MODE_OUTPUT) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) mma(O[rt], lds_frag<OP>(sQh, LDK, rt * 16, kb * 32), mf);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (MODE == MODE_OUTPUT) {
          // O = diag(gamma) Q M0 + P V_new
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[rt][i] *= sGam[rt * 16 + 4 * g4 + i];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const Frag<OP> vn = acc_frag<OP>(U[cw][2 * kb], U[cw][2 * kb + 1]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
              if (kb * 32 <= rt * 16 + 15) mma(O[rt], lds_frag<OP>(sP, LC, rt * 16, kb * 32), vn);
            __builtin_amdgcn_sched_barrier(0);
          }
          store_o(O, ct, t0, n, Ex[cw]);
        }
        // M <- gamma_C M + K^T diag(e^{g_C - g}) V_new
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          Frag<OP> vd;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vd.v[j] = from_f32<OP>(U[cw][2 * kb][j] * sDec[kb * 32 + 4 * g4 + j]);
            vd.v[4 + j] = from_f32<OP>(U[cw][2 * kb + 1][j] * sDec[kb * 32 + 16 + 4 * g4 + j]);
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            if (kb == 0) {
#pragma unroll
              for (int i = 0; i < 4; ++i) Macc[cw][rt][i] *= gamC;
            }
            mma(Macc[cw][rt], lds_frag<OP>(sKt, LC, rt * 16, kb * 32), vd);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Each A fragment (rows of W, Q, P, K^T) is read from LDS once and applied
      // to all of the wave's column tiles.
      bool has[CPW];  // the wave owns column tile wave + cw * NWAVE
#pragma unroll
      for (int cw = 0; cw < CPW; ++cw) has[cw] = wave + cw * NWAVE < NCT;
      // V_new = U0 - W M0 and (outputs) Q M0
      f4_t O[MODE == MODE_OUTPUT ? CPW : 1][4];
#pragma unroll
      for (int cw = 0; cw < (MODE == MODE_OUTPUT ? CPW : 1); ++cw)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) O[cw][rt] = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        Frag<OP> mf[CPW];
#pragma unroll
        for (int cw = 0; cw < CPW; ++cw) mf[cw] = acc_frag<OP>(Macc[cw][2 * kb], Macc[cw][2 * kb + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const Frag<OP> aw = lds_frag<OP>(sW, LDK, rt * 16, kb * 32);
#pragma unroll
          for (int cw = 0; cw < CPW; ++cw)
            if (has[cw]) mma(U[cw][rt], aw, mf[cw]);
          if (MODE == MODE_OUTPUT) {
            const Frag<OP> aq = lds_frag<OP>(sQh, LDK, rt * 16, kb * 32);
#pragma unroll
            for (int cw = 0; cw < CPW; ++cw)
              if (has[cw]) mma(O[cw][rt], aq, mf[cw]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (MODE == MODE_OUTPUT) {
        // O = diag(gamma) Q M0 + P V_new
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gm = sGam[rt * 16 + 4 * g4 + i];
#pragma unroll
            for (int cw = 0; cw < CPW; ++cw) O[cw][rt][i] *= gm;
          }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          Frag<OP> vn[CPW];
#pragma unroll
          for (int cw = 0; cw < CPW; ++cw) vn[cw] = acc_frag<OP>(U[cw][2 * kb], U[cw][2 * kb + 1]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
            if (kb * 32 <= rt * 16 + 15) {
              const Frag<OP> ap = lds_frag<OP>(sP, LC, rt * 16, kb * 32);
#pragma unroll
              for (int cw = 0; cw < CPW; ++cw)
                if (has[cw]) mma(O[cw][rt], ap, vn[cw]);
            }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int cw = 0; cw < CPW; ++cw)
          if (has[cw]) store_o(O[cw], wave + cw * NWAVE, t0, n, Ex[cw]);
      }
      // M <- gamma_C M + K^T diag(e^{g_C - g}) V_new
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<OP> vd[CPW];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d0 = sDec[kb * 32 + 4 * g4 + j], d1 = sDec[kb * 32 + 16 + 4 * g4 + j];
#pragma unroll
          for (int cw = 0; cw < CPW; ++cw) {
            vd[cw].v[j] = from_f32<OP>(U[cw][2 * kb][j] * d0);
            vd[cw].v[4 + j] = from_f32<OP>(U[cw][2 * kb + 1][j] * d1);
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const Frag<OP> ak = lds_frag<OP>(sKt, LC, rt * 16, kb * 32);
#pragma unroll
          for (int cw = 0; cw < CPW; ++cw)
            if (has[cw]) {
              if (kb == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) Macc[cw][rt][i] *= gamC;
              }
              mma(Macc[cw][rt], ak, vd[cw]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // (no barrier here: the next chunk's first LDS write follows the barrier
    // at the top of the loop, which every wave reaches only after its column phase)
  }

  // ---- results
#pragma unroll
  for (int cw = 0; cw < CPW; ++cw) {
    const int ct = wave + cw * NWAVE;
    if (ct >= NCT) continue;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + 4 * g4 + i;
        const float mv = SCALED ? ldexpf(Macc[cw][rt][i], held_exp(Ex[cw])) : Macc[cw][rt][i];  // true units
        if (MODE == MODE_OUTPUT) {
          if (s == nseg_b - 1) a.S_final[(bh * DK + row) * DV + ct * 16 + m16] = mv;
        } else if (MODE == MODE_CKPT) {
        } else if (ct < VCT) {
          a.Dsum[((bh * a.nseg + s) * DK + row) * DV + ct * 16 + m16] = mv;
        } else {
          a.Phi[((bh * a.nseg + s) * DK + row) * DK + (ct - VCT) * 16 + m16] = mv;
        }
      }
  }
}


// ------------------------------------------------------------ segment scan

// fp16 split products: x ~= hi + lo with both parts fp16, three products
// keep about 22 bits of the fp32 operands.
__device__ __forceinline__ void split_mma(f4_t& acc, const float* av, const float* bv, _Float16) {
  Frag<_Float16> ah, al, bh, bl;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ah.v[j] = (_Float16)av[j];
    al.v[j] = (_Float16)(av[j] - (float)ah.v[j]);
    bh.v[j] = (_Float16)bv[j];
    bl.v[j] = (_Float16)(bv[j] - (float)bh.v[j]);
  }
  mma(acc, ah, bh);
  mma(acc, ah, bl);
  mma(acc, al, bh);
}

__device__ __forceinline__ void split_mma(f4_t& acc, const float* av, const float* bv, float) {
  Frag<float> af, bf;
#pragma unroll
  for (int j = 0; j < 8; ++j) { af.v[j] = av[j]; bf.v[j] = bv[j]; }
  mma(acc, af, bf);
}

// grid (DV/16, H, B), one wave per row tile of M (DK/16 waves): M_0 = S0 (or
// 0); M_{s+1} = Phi_s M_s + D_s over the segments of sequence b (nseg is the
// per-sequence stride of the segment buffers; a packed batch's shorter
// sequences use fewer).  Wave w forms row tile w of each M from the whole
// previous M, which the waves share through LDS; each wave's D_s and Phi_s
// rows of the next two segments load while it multiplies.
template <int DK, int DV, typename OP>
__global__ __launch_bounds__(DK / 16 * WAVE) void scan_kernel(int H, int nseg, const int* cu_seqlens, int Tmax,
                                                              int64_t total, int seg_len, const float* S0, const float* Dsum,
                                                              const float* Phi, float* Mstart) {
  constexpr int KB = DK / 32, LM = 16 + 1;
  __shared__ float sM[DK * LM];  // M, [DK][16] (+1 pad)
  const int ct = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int64_t tok0;
  int T;
  seq_span(cu_seqlens, Tmax, total, b, tok0, T);
  const int nseg_b = seq_segments(T, seg_len);
  const int rt = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int m16 = lane & 15, g4 = lane >> 4;
  const int64_t bh = (int64_t)b * H + h;
  const int col = ct * 16 + m16;
  f4_t M;
#pragma unroll
  for (int i = 0; i < 4; ++i) M[i] = S0 ? S0[(bh * DK + rt * 16 + 4 * g4 + i) * DV + col] : 0.f;
  auto load_step = [&](int s, float (&d)[4], float (&pm)[KB][8]) {
    const float* D = Dsum + (bh * nseg + s) * DK * DV;
    const float* P = Phi + (bh * nseg + s) * DK * DK;
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = D[(rt * 16 + 4 * g4 + i) * DV + col];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const float* prow = P + (rt * 16 + m16) * DK + kb * 32 + 4 * g4;
#pragma unroll
      for (int j = 0; j < 4; ++j) { pm[kb][j] = prow[j]; pm[kb][4 + j] = prow[16 + j]; }
    }
  };
  const int last = nseg_b - 1;  // M_last is stored, not advanced
  // the maps of the next two segments are in flight while one multiplies: three
  // register buffers in rotation, the loop unrolled by three so that no buffer
  // is copied (a copy would wait for its loads)
  float d0[4], p0[KB][8], d1[4], p1[KB][8], d2[4], p2[KB][8];
  if (last > 0) load_step(0, d0, p0);
  if (last > 1) load_step(1, d1, p1);
  // step s from the buffer (dc, pc), then the segment s + 2 into (dl, pl);
  // returns false once M_last is stored
  auto step = [&](int s, const float (&dc)[4], const float (&pc)[KB][8], float (&dl)[4], float (&pl)[KB][8]) {
    float* dst = Mstart + (bh * nseg + s) * DK * DV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[(rt * 16 + 4 * g4 + i) * DV + col] = M[i];
      sM[(rt * 16 + 4 * g4 + i) * LM + m16] = M[i];
    }
    if (s == last) return false;
    if (s + 2 < last) load_step(s + 2, dl, pl);
    __syncthreads();  // every row tile of M_s is in LDS
    // B fragments: rows kb*32 + kperm(g, j) of M_s, this lane's column
    f4_t acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = dc[i];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float bv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) bv[j] = sM[(kb * 32 + kperm(g4, j)) * LM + m16];
      split_mma(acc, pc[kb], bv, OP());
    }
    M = acc;
    __syncthreads();  // every wave has read M_s before it is overwritten
    return true;
  };
  for (int s = 0;; s += 3) {
    if (!step(s, d0, p0, d2, p2)) break;
    if (!step(s + 1, d1, p1, d0, p0)) break;
    if (!step(s + 2, d2, p2, d1, p1)) break;
  }
}

// ------------------------------------------------------------ prologue hook

// grid (nchunks, H, B), 512 threads: the chunk kernels' prologue on its own.
template <int DK, typename IO>
__global__ __launch_bounds__(PRO_THR) void prologue_kernel(int T, int H, const IO* q, const IO* k,
                                                           const float* alpha, float* qhat, float* khat,
                                                           float* gout) {
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = c * C, n = min(C, T - t0);
  Prologue<DK, IO> pr;
  pr.load(q, k, ((int64_t)b * T + t0) * H + h, H, n, true);
  pr.finish(true);
  if (pr.row < n) {
    const int64_t off = (((int64_t)b * T + t0 + pr.row) * H + h) * DK + pr.part * Prologue<DK, IO>::E;
#pragma unroll
    for (int e = 0; e < Prologue<DK, IO>::E; ++e) {
      khat[off + e] = pr.kv[e];
      qhat[off + e] = pr.qv[e];
    }
  }
  if (threadIdx.x < WAVE) {
    const int row = threadIdx.x;
    const int64_t idx = ((int64_t)b * T + t0 + row) * H + h;
    const float g = chunk_gate_scan(row < n ? alpha[idx] : 1.f);
    if (row < n) gout[idx] = g * 0.69314718055994531f;  // back to natural log
  }
}

// ------------------------------------------------------------ host side

PrefillPlan plan_prefill(int B, int T, int H, int dk, int dv, int io, int out, int seg_len) {
  PrefillPlan p{};
  p.B = B; p.T = T; p.H = H; p.dk = dk; p.dv = dv; p.io = io; p.out = out;
  p.tokens = (int64_t)B * T;
  p.cu_seqlens = nullptr;
  p.nchunks = (int)(((int64_t)T + C - 1) / C);
  if (p.nchunks == 0) { p.seg_len = 1; p.nseg = 0; return p; }
  if (seg_len <= 0) {
    const int64_t units = (int64_t)B * H;
    int nseg = units >= NCU ? 1 : (int)(NCU / units);
    if (nseg > p.nchunks) nseg = p.nchunks;
    if (nseg < 1) nseg = 1;
    seg_len = (p.nchunks + nseg - 1) / nseg;
  }
  p.seg_len = seg_len;
  p.nseg = (p.nchunks + seg_len - 1) / seg_len;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t taps_bytes(const PrefillPlan& p) { return align256((size_t)p.tokens * p.H * 4 * sizeof(float)); }

// (several segments) Mstart, Dsum, Phi
static size_t segment_bytes(const PrefillPlan& p) {
  if (p.nseg <= 1) return 0;
  const size_t st = (size_t)p.B * p.H * p.nseg;
  return 2 * align256(st * p.dk * p.dv * sizeof(float)) + align256(st * p.dk * p.dk * sizeof(float));
}

size_t prefill_base_bytes(const PrefillPlan& p) { return taps_bytes(p) + segment_bytes(p); }
size_t prefill_workspace_bytes(const PrefillPlan& p) { return prefill_base_bytes(p); }
size_t prefill_static_workspace_bytes(const PrefillPlan& p) { return segment_bytes(p); }

template <int DK, int DV, typename IO, typename OP, typename OUT, bool SC>
static hipError_t run_prefill(const PrefillPlan& p, ChunkArgs a, hipStream_t stream) {
  const dim3 blk(NTHR);
  if (p.nseg > 1) {
    chunk_kernel<DK, DV, IO, OP, OUT, MODE_SUMMARY, SC><<<dim3(p.nseg - 1, p.H, p.B), blk, 0, stream>>>(a);
    scan_kernel<DK, DV, float><<<dim3(DV / 16, p.H, p.B), dim3(DK / 16 * WAVE), 0, stream>>>(
        p.H, p.nseg, a.cu_seqlens, a.T, a.total, a.seg_len, a.S0, a.Dsum, a.Phi, const_cast<float*>(a.Mstart));
  }
  chunk_kernel<DK, DV, IO, OP, OUT, MODE_OUTPUT, SC><<<dim3(p.nseg, p.H, p.B), blk, 0, stream>>>(a);
  return hipGetLastError();
}

template <int DK, int DV, typename IO, typename OP, bool SC = false>
static hipError_t run_prefill_out(const PrefillPlan& p, ChunkArgs a, hipStream_t stream) {
  return p.out == IO_F32 ? run_prefill<DK, DV, IO, OP, float, SC>(p, a, stream)
                         : run_prefill<DK, DV, IO, OP, bf16_t, SC>(p, a, stream);
}

static void set_segment_buffers(const PrefillPlan& p, ChunkArgs& a, char* ws) {
  if (p.nseg <= 1) return;
  const size_t st = (size_t)p.B * p.H * p.nseg;
  a.Mstart = reinterpret_cast<float*>(ws);
  ws += align256(st * p.dk * p.dv * sizeof(float));
  a.Dsum = reinterpret_cast<float*>(ws);
  ws += align256(st * p.dk * p.dv * sizeof(float));
  a.Phi = reinterpret_cast<float*>(ws);
}

#define JB_PREFILL_BF16_CASES(X) \
  X(32, 64) X(32, 128) X(32, 256) X(64, 64) X(64, 128) X(64, 256) \
  X(96, 64) X(96, 128) X(96, 256) X(128, 64) X(128, 128) X(128, 256)
#define JB_PREFILL_F32_CASES(X) X(32, 64) X(64, 64)

// the segment scan on its own (the fused passes' summaries feed it)
static hipError_t launch_scan(const PrefillPlan& p, const ChunkArgs& a, hipStream_t stream) {
#define CASE(DK_, DV_)                                                                                       \
  if (p.dk == DK_ && p.dv == DV_) {                                                                          \
    scan_kernel<DK_, DV_, float><<<dim3(DV_ / 16, p.H, p.B), dim3(DK_ / 16 * WAVE), 0, stream>>>(              \
        p.H, p.nseg, a.cu_seqlens, a.T, a.total, a.seg_len, a.S0, a.Dsum, a.Phi, const_cast<float*>(a.Mstart)); \
    return hipGetLastError();                                                                                \
  }
  JB_PREFILL_BF16_CASES(CASE)
#undef CASE
  return hipErrorInvalidValue;
}

bool prefill_supported(const PrefillPlan& p) {
#define CASE(DK_, DV_) if (p.dk == DK_ && p.dv == DV_) return true;
  if (p.io == IO_BF16) { JB_PREFILL_BF16_CASES(CASE) }
  else { JB_PREFILL_F32_CASES(CASE) }
#undef CASE
  return false;
}

hipError_t launch_prefill(const PrefillPlan& p, const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, const float* taps,
                          const void* conv_in, const float* S0, void* o, float* S_final,
                          void* workspace, hipStream_t stream) {
  if (p.nchunks == 0) return hipSuccess;
  ChunkArgs a{};
  a.T = p.T; a.H = p.H; a.nchunks = p.nchunks; a.seg_len = p.seg_len; a.nseg = p.nseg;
  a.cu_seqlens = p.cu_seqlens;
  a.total = p.tokens;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.taps = taps; a.conv_in = conv_in;
  a.S0 = S0; a.o = o; a.S_final = S_final;
  set_segment_buffers(p, a, static_cast<char*>(workspace) + taps_bytes(p));
  if (p.io == IO_BF16 && fwd_supported(p.dk, p.dv)) {
    // the fused chunk passes: summaries, scan, outputs
    FwdArgs f{};
    f.T = p.T; f.H = p.H; f.seg_len = p.seg_len; f.nseg = p.nseg; f.cu_seqlens = p.cu_seqlens; f.total = p.tokens;
    f.q = static_cast<const uint16_t*>(q); f.k = static_cast<const uint16_t*>(k);
    f.v = static_cast<const uint16_t*>(v); f.conv_in = static_cast<const uint16_t*>(conv_in);
    f.alpha = alpha; f.beta = beta; f.taps = taps; f.S0 = S0; f.Mstart = a.Mstart; f.Dsum = a.Dsum; f.Phi = a.Phi;
    f.o = o; f.S_final = S_final;
    hipError_t e = hipSuccess;
    if (p.nseg > 1) {
      e = launch_fwd(f, 1, p.dk, p.dv, p.out == IO_BF16, p.nseg, p.H, p.B, stream);
      if (e == hipSuccess) e = launch_scan(p, a, stream);
    }
    if (e == hipSuccess) e = launch_fwd(f, 2, p.dk, p.dv, p.out == IO_BF16, p.nseg, p.H, p.B, stream);
    return e;
  }
  // (every bf16 shape has the fused passes; the chunk kernel serves the all-fp32 mode)
#define CASE(DK_, DV_) \
  if (p.dk == DK_ && p.dv == DV_) return run_prefill_out<DK_, DV_, float, float>(p, a, stream);
  if (p.io == IO_F32) { JB_PREFILL_F32_CASES(CASE) }
#undef CASE
  return hipErrorInvalidValue;
}

#define JB_PREFILL_STATIC_CASES(X) X(32, 64) X(64, 128) X(96, 256) X(128, 256)

bool prefill_static_supported(const PrefillPlan& p) {
#define CASE(DK_, DV_) if (p.dk == DK_ && p.dv == DV_) return true;
  if (p.io == IO_BF16) { JB_PREFILL_STATIC_CASES(CASE) }
#undef CASE
  return false;
}

hipError_t launch_prefill_static(const PrefillPlan& p, const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta, const float* wq, const float* wk,
                                 const float* wv, const void* cq_in, const void* ck_in, const void* cv_in,
                                 const float* S0, void* o, float* S_final, void* workspace, hipStream_t stream) {
  if (p.nchunks == 0) return hipSuccess;
  ChunkArgs a{};
  a.T = p.T; a.H = p.H; a.nchunks = p.nchunks; a.seg_len = p.seg_len; a.nseg = p.nseg;
  a.cu_seqlens = p.cu_seqlens;
  a.total = p.tokens;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.conv_in = cv_in;
  a.wq = wq; a.wk = wk; a.wv = wv; a.cq_in = cq_in; a.ck_in = ck_in;
  a.S0 = S0; a.o = o; a.S_final = S_final;
  set_segment_buffers(p, a, static_cast<char*>(workspace));
#define CASE(DK_, DV_) \
  if (p.dk == DK_ && p.dv == DV_) return run_prefill_out<DK_, DV_, bf16_t, _Float16, true>(p, a, stream);
  if (p.io == IO_BF16) { JB_PREFILL_STATIC_CASES(CASE) }
#undef CASE
  return hipErrorInvalidValue;
}

template <int DK, int DV>
static hipError_t run_ckpt(const PrefillPlan& p, ChunkArgs a, hipStream_t stream) {
  const dim3 blk(NTHR);
  if (p.nseg > 1) {
    chunk_kernel<DK, DV, bf16_t, _Float16, float, MODE_SUMMARY, false><<<dim3(p.nseg - 1, p.H, p.B), blk, 0, stream>>>(a);
    scan_kernel<DK, DV, float><<<dim3(DV / 16, p.H, p.B), dim3(DK / 16 * WAVE), 0, stream>>>(
        p.H, p.nseg, a.cu_seqlens, a.T, a.total, a.seg_len, a.S0, a.Dsum, a.Phi, const_cast<float*>(a.Mstart));
  }
  chunk_kernel<DK, DV, bf16_t, _Float16, float, MODE_CKPT, false><<<dim3(p.nseg, p.H, p.B), blk, 0, stream>>>(a);
  return hipGetLastError();
}

#define JB_BACKWARD_CASES(X) X(32, 64) X(64, 128) X(96, 256) X(128, 256)

bool backward_supported(int io, int dk, int dv) {
#define CASE(DK_, DV_) if (dk == DK_ && dv == DV_) return true;
  if (io == IO_BF16) { JB_BACKWARD_CASES(CASE) }
#undef CASE
  return false;
}

hipError_t launch_prefill_ckpt(const PrefillPlan& p, const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, const float* taps, const void* conv_in, const float* S0,
                               _Float16* Mck, char* img, void* workspace, hipStream_t stream,
                               const float* ck_scale) {
  if (p.nchunks == 0) return hipSuccess;
  ChunkArgs a{};
  a.T = p.T; a.H = p.H; a.nchunks = p.nchunks; a.seg_len = p.seg_len; a.nseg = p.nseg;
  a.total = p.tokens;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.taps = taps; a.conv_in = conv_in;
  a.S0 = S0; a.Mck = Mck; a.img = img; a.ck_scale = ck_scale;
  set_segment_buffers(p, a, static_cast<char*>(workspace) + taps_bytes(p));
#define CASE(DK_, DV_) \
  if (p.dk == DK_ && p.dv == DV_) return run_ckpt<DK_, DV_>(p, a, stream);
  if (p.io == IO_BF16) { JB_BACKWARD_CASES(CASE) }
#undef CASE
  return hipErrorInvalidValue;
}

hipError_t launch_prologue(int io, int B, int T, int H, int dk, const void* q, const void* k,
                           const float* alpha, float* qhat, float* khat, float* g, hipStream_t stream) {
  const int nch = (T + C - 1) / C;
  if (nch == 0 || B == 0) return hipSuccess;
  const dim3 grid(nch, H, B), blk(PRO_THR);
#define CASE(DK_)                                                                                   \
  if (dk == DK_) {                                                                                  \
    if (io == IO_BF16)                                                                              \
      prologue_kernel<DK_, bf16_t><<<grid, blk, 0, stream>>>(T, H, (const bf16_t*)q, (const bf16_t*)k, \
                                                             alpha, qhat, khat, g);                 \
    else                                                                                            \
      prologue_kernel<DK_, float><<<grid, blk, 0, stream>>>(T, H, (const float*)q, (const float*)k, \
                                                            alpha, qhat, khat, g);                  \
    return hipGetLastError();                                                                       \
  }
  CASE(32) CASE(64) CASE(96) CASE(128)
#undef CASE
  return hipErrorInvalidValue;
}

}  // namespace jb
