// jb_fwd.hip -- the chunked JetBlock prefill for bf16 inputs, one fused pass
// per segment.
//
// The recurrence and its chunked (WY/UT) form are those of jb_prefill.hip
// (Gated DeltaNet time mixing: Jet-Nemotron csdn translation, section 2.4;
// dynamic causal conv of the values, section 2.4 and the xugj520 blog,
// section 2.2).  A long sequence is cut into segments; the summary pass runs
// each segment but the last from the zero state on augmented columns [D | Phi]
// (Phi starting at I), the scan chains the segment maps, and the output pass
// reruns every segment from its true start state.  Each pass forms every
// chunk's state-independent tiles from the raw q, k, v rows itself, so the only
// HBM traffic is the compulsory inputs (read twice for all but the last
// segment) and o.
//
// Workgroup: one per (segment, head, sequence); wave w owns the 16-column
// tiles w, w + 8, .. of the state (value columns, and in the summary the
// transition columns after them), held in fp32 accumulators at a per-tile
// power-of-two scale (jb_chunk.h).  Per chunk of C = 64 tokens:
//   A  normalise the staged q, k rows into K^, Q^ (fp16);
//   B  Gram tiles K^K^T and Q^K^T -> -A, its fp32 diagonal blocks, P (written
//      as whole rows: each product is formed transposed); waves 4..7 invert
//      the four 16x16 diagonal blocks of I + A; every wave forms its
//      right-hand sides diag(b) V' = Band V_ext on the bf16 matrix cores,
//      picks its tiles' exponents and subtracts diag(b gamma) K^ M (output
//      pass: also Q^ M);
//   D  T = (I + A)^{-1} by blocked forward substitution on the matrix cores
//      (waves 0..3, a column block each); the gate wave scans the next
//      chunk's gates and writes its conv band;
//   E  V_new = T R, O = diag(gamma) Q^ M + P V_new (staged in LDS, stored at
//      the start of the next chunk), and M <- gamma_C M + K^T diag(e^{g_C - g}) V_new.
// The next chunk's q and k rows move into LDS by DMA from phase B on, its
// value rows from phase D on, and the gate rows two chunks ahead, so their
// HBM latency overlaps the chunk.
//
// Operands read down a column of a row-major tile (K^ as K^T, -W^T as W, the
// value rows) come from ds_read_b64_tr_b16: within each group of 16 lanes,
// lane 4a + b receives element b of the 8-byte pieces addressed by lanes
// 4j + a (j = 0..3), so one instruction yields four K values of a fragment.
#include <algorithm>

#include "jb_chunk.h"
#include "jb_device.h"
#include "jb_frag.h"
#include "jb_internal.h"

namespace jb {
namespace fwd {

enum { SUMMARY = 0, OUTPUT = 1 };

// the blocked triangular solve of jb_chunk.h on these fragments, Y = (I + A)^{-1} Y,
// from the kperm row bases of -A (row stride LC) and of the diagonal-block
// inverses (LLI, columns 16..31 zero)
template <int LC, int LLI>
__device__ __forceinline__ void solve(f4_t (&Y)[4], const _Float16* bAn, const _Float16* bLi) {
  const f4_t z = zero4();
  Y[0] = mfma(row_frag_kp<LLI>(bLi, 0, 0), acc_frag2(Y[0], z), z);
  Y[1] = mfma(row_frag_kp<LC>(bAn, 16, 0), acc_frag2(Y[0], z), Y[1]);
  Y[1] = mfma(row_frag_kp<LLI>(bLi, 16, 0), acc_frag2(Y[1], z), z);
  const half8_t f01 = acc_frag2(Y[0], Y[1]);
  Y[2] = mfma(row_frag_kp<LC>(bAn, 32, 0), f01, Y[2]);
  Y[3] = mfma(row_frag_kp<LC>(bAn, 48, 0), f01, Y[3]);
  Y[2] = mfma(row_frag_kp<LLI>(bLi, 32, 0), acc_frag2(Y[2], z), z);
  Y[3] = mfma(row_frag_kp<LC>(bAn, 48, 32), acc_frag2(Y[2], z), Y[3]);
  Y[3] = mfma(row_frag_kp<LLI>(bLi, 48, 0), acc_frag2(Y[3], z), z);
}

// ------------------------------------------------------------ geometry

template <int DK, int DV, int MODE>
struct Geo {
  static constexpr bool OUTM = MODE == OUTPUT;
  static constexpr int NCT = OUTM ? DV / 16 : (DV + DK) / 16;  // column tiles
  static constexpr int VCT = DV / 16;                          // value column tiles
  static constexpr int RT = DK / 16, KB = DK / 32;
  static constexpr int NW = 8;                                 // waves
  static constexpr int TPW = (NCT + NW - 1) / NW;              // tiles per wave: wave w owns w, w + 8, ..
  static constexpr int GW = NW - 1;                            // gate wave
  static constexpr int IW = NW - 2;                            // inverse wave
  static constexpr int LDK = DK + 8, LC = C + 8, LTT = C + 16, LAD = 20, LLI = 36, LT = 40;
  // value rows in groups of VRPG rows (1 KB, one full-wave DMA), 32 bytes of
  // padding after each group; row r at vrow(r).  Within row j of a group the
  // 16-column tiles are XOR-permuted by vsw(j) (< NW), so that the 8 rows one
  // half-wave reads down a column tile fall in distinct 32-byte bank slots.
  static constexpr int VRPG = 1024 / (DV * 2), VG = 1024 + 32, NVG = (C + 3 + VRPG - 1) / VRPG;
  static constexpr int vrow(int r) { return (r / VRPG) * VG + (r % VRPG) * DV * 2; }
  static constexpr int vsw(int j) { return DV == 256 ? 4 * j : DV == 128 ? 2 * j : j >> 1; }
  static constexpr int a16(int x) { return (x + 15) / 16 * 16; }
  static constexpr int oG = 0;                                  // g, gamma, beta, e^{g_C - g}: [2][4][C] f32
  static constexpr int oT = oG + 2 * 4 * C * 4;                 // band: [hi, lo][4][16][LT] bf16
  static constexpr int oKh = a16(oT + 2 * 4 * 16 * LT * 2);     // [C][LDK] K^
  static constexpr int szQh = OUTM ? C * LDK * 2 : 0;
  static constexpr int szT = C * LTT * 2;
  static constexpr int oQW = a16(oKh + C * LDK * 2);            // Q^ (output), then T^T [C][LTT]
  static constexpr int oAn = a16(oQW + (szQh > szT ? szQh : szT));  // [C][LC] -A
  static constexpr int oAd = a16(oAn + C * LC * 2);             // [C][LAD] f32 diagonal blocks of A
  static constexpr int oLi = a16(oAd + C * LAD * 4);            // [C][LLI] their inverses
  static constexpr int oP = a16(oLi + C * LLI * 2);             // [C][LC] P (output)
  static constexpr int oSO = oAn;                               // (output) o rows of a chunk, bf16 [C][DV]
  static constexpr int SO_END = oSO + (OUTM ? C * DV * 2 : 0);  // over -A .. P, dead once P V_new is done
  static constexpr int WORK0 = a16(oP + (OUTM ? C * LC * 2 : 0));
  static constexpr int WORK = WORK0 > SO_END ? WORK0 : a16(SO_END);
  static constexpr int STAGE = (OUTM ? 2 : 1) * C * DK * 2 + 2 * C * 6 * 4 + NVG * VG;
  static_assert(WORK + STAGE <= 160 * 1024, "LDS budget of one CU exceeded");
  static_assert(RT <= NW, "one wave per W column tile");
  static_assert((LDK * 2) % 16 == 0 && VG % 16 == 0 && (LC * 2) % 8 == 0 && (LTT * 2) % 8 == 0, "aligned rows");
  static_assert(16 % VRPG == 0 && VRPG * DV * 2 == 1024, "value row groups of 1 KB that tile 16-row windows");
  static_assert(vsw(VRPG - 1) < NW && vsw(VRPG - 1) < VCT && (NW & (NW - 1)) == 0,
                "tile swizzle within a row, commuting with the wave stride of column tiles");
};

// ------------------------------------------------------------ kernel

template <int DK, int DV, typename OUT, int MODE>
__global__ __launch_bounds__(512, 1) void fwd_kernel(FwdArgs a) {
  using G = Geo<DK, DV, MODE>;
  constexpr bool OUTM = G::OUTM;
  // bf16 outputs leave through LDS as whole rows (one 16-byte piece per lane,
  // a chunk row in contiguous lanes); f32 outputs straight from the registers
  constexpr bool STAGE_O = OUTM && sizeof(OUT) == 2;
  constexpr int NCT = G::NCT, VCT = G::VCT, RT = G::RT, KB = G::KB, NW = G::NW, TPW = G::TPW;
  constexpr int LDK = G::LDK, LC = G::LC, LTT = G::LTT, LAD = G::LAD, LLI = G::LLI, LT = G::LT;
  constexpr int VRPG = G::VRPG, VG = G::VG, NVG = G::NVG;

  // working tiles, and the DMA staging areas as arrays of their own (so the
  // compiler can tell that reads of the tiles never wait on the DMA)
  __shared__ __attribute__((aligned(16))) char work[G::WORK];
  __shared__ __attribute__((aligned(16))) bf16_t sKr[C * DK];
  __shared__ __attribute__((aligned(16))) bf16_t sQr[OUTM ? C * DK : 8];
  __shared__ __attribute__((aligned(16))) float sGr[2 * C * 6];  // [chunk & 1]: alpha [C], beta [C], taps [C][4]
  __shared__ __attribute__((aligned(16))) char sV[NVG * VG];
  float* sG2 = reinterpret_cast<float*>(work + G::oG);  // [chunk & 1]: g, gamma, beta, e^{g_C - g}
  bf16_t* sT = reinterpret_cast<bf16_t*>(work + G::oT);
  _Float16* sKh = reinterpret_cast<_Float16*>(work + G::oKh);
  _Float16* sQh = reinterpret_cast<_Float16*>(work + G::oQW);
  _Float16* sAn = reinterpret_cast<_Float16*>(work + G::oAn);
  float* sAd = reinterpret_cast<float*>(work + G::oAd);
  _Float16* sLi = reinterpret_cast<_Float16*>(work + G::oLi);
  _Float16* sP = reinterpret_cast<_Float16*>(work + G::oP);
  // the same tiles as LDS addresses, for the transposed reads and the DMA
  const lds_char* lKh = (const lds_char*)work + G::oKh;
  const lds_char* lTt = (const lds_char*)work + G::oQW;  // T^T [C][LTT]
  const lds_char* lV = (const lds_char*)sV;
  lds_char* lKr = (lds_char*)sKr;
  lds_char* lQr = (lds_char*)sQr;
  lds_char* lGr = (lds_char*)sGr;
  lds_char* lVw = (lds_char*)sV;

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = a.H;
  int64_t tok0;
  int T;
  seq_span(a.cu_seqlens, a.T, a.total, b, tok0, T);
  const int nseg_b = seq_segments(T, a.seg_len);
  if (s >= (OUTM ? nseg_b : nseg_b - 1)) return;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // (the block has NW waves: with this known, which tiles a wave owns and how
  // many o stores it issues per chunk are compile-time facts, and the compiler
  // can count the DMA transfers complete at the top wait; the summary pass
  // stores nothing per chunk and waits for everything there)
  if constexpr (OUTM) __builtin_assume(wave >= 0 && wave < NW);
  const int m16 = lane & 15, g4 = lane >> 4;
  const bf16_t* q = a.q;
  const bf16_t* k = a.k;
  const bf16_t* v = a.v;
  const bf16_t* cin = a.conv_in;
  const int64_t bh = (int64_t)b * H + h;
  // column tile cw of this wave: wave + 8 cw; value tiles have right-hand sides
  auto tile = [&](int cw) { return wave + cw * NW; };
  auto has = [&](int cw) { return wave + cw * NW < NCT; };
  auto isval = [&](int cw) { return wave + cw * NW < VCT; };

  // this lane's bases in the tiles
  const lds_char* tKkp = tr_base_kp(lKh, LDK);   // K^ down its columns (K^T, for the state update)
  const lds_char* tTkp = tr_base_kp(lTt, LTT);   // T^T down its columns (T)
  // value rows down their columns (the kperm lane rows of tr_base_kp, in the
  // grouped row layout): windows from a multiple of 16, and the last one from row C + 3 - 32
  // (tile wave + NW cw of row r sits at tile (wave ^ vsw(r % VRPG)) + NW cw)
  const int vx = 4 * (lane >> 4) + ((lane >> 2) & 3), va = 8 * (lane & 3);
  const lds_char* tVa = lV + opaque(G::vrow(vx) + 32 * (wave ^ G::vsw(vx % VRPG)) + va);
  const lds_char* tVb =
      lV + opaque(G::vrow(C + 3 - 32 + vx) + 32 * (wave ^ G::vsw((C + 3 - 32 + vx) % VRPG)) + va);
  const _Float16* rKct = row_base_ct(sKh, LDK);  // rows of K^, Q^ (Gram tiles)
  const _Float16* rQct = row_base_ct(sQh, LDK);
  const _Float16* rQkp = row_base_kp(sQh, LDK);  // rows of Q^ (Q^ M)
  const _Float16* rKkp = row_base_kp(sKh, LDK);  // rows of K^ (K^ M)
  const _Float16* rPkp = row_base_kp(sP, LC);
  const _Float16* rAkp = row_base_kp(sAn, LC);
  const _Float16* rLkp = row_base_kp(sLi, LLI);
  const _Float16* rTkp = row_base_kp(reinterpret_cast<const _Float16*>(sT), LT);  // band rows (bf16 bits)

  // ---- initial state, accumulator layout: lane holds M[16 rt + 4 g + i][16 ct + m16]
  f4_t Macc[TPW][RT];
  int Ex[TPW];
#pragma unroll
  for (int cw = 0; cw < TPW; ++cw) {
    const int ct = tile(cw);
    Ex[cw] = E_FRESH;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      Macc[cw][rt] = zero4();
      if (!has(cw)) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + 4 * g4 + i;
        if (!OUTM) {
          if (ct >= VCT) Macc[cw][rt][i] = (row == (ct - VCT) * 16 + m16) ? 1.f : 0.f;
        } else {
          const float* src = a.nseg > 1 ? a.Mstart + ((bh * a.nseg + s) * DK) * DV
                                        : (a.S0 ? a.S0 + bh * DK * DV : nullptr);
          Macc[cw][rt][i] = src ? src[row * DV + ct * 16 + m16] : 0.f;
        }
      }
    }
  }

  // tiles not rewritten per chunk: the band outside its diagonals, P above its
  // block diagonal (but see the o staging below)
  for (int e = tid; e < 2 * 4 * 16 * LT / 8; e += NW * 64)
    reinterpret_cast<uint4*>(sT)[e] = make_uint4(0u, 0u, 0u, 0u);
  if (OUTM)
    for (int e = tid; e < C * C; e += NW * 64) {
      const int r = e / C, c = e % C;
      if ((c >> 4) > (r >> 4)) sP[r * LC + c] = (_Float16)0.f;
    }

  const int c_begin = s * a.seg_len;
  const int c_end = min((T + C - 1) / C, c_begin + a.seg_len);

  // ---- raw inputs of chunk cc into the staging areas by DMA (a buffer
  // resource per chunk and stream, per-lane 32-bit byte offsets); rows past
  // the sequence are left as they are (the prologue masks them) except the
  // value rows, which are zeroed (the band multiplies them by zero
  // coefficients, and stale values could be non-finite)
  const uint32_t rowq = (uint32_t)(H * DK * 2), rowv = (uint32_t)(H * DV * 2);  // bytes between tokens
  // q, k and gate rows of chunk cc, shared by waves 0 .. nw - 1 (wave wv takes
  // the 64-piece rows wv, wv + nw, ..; the last of them also the gates)
  auto issue_qkg = [&](int cc, int wv, int nw) {
    const int t0c = cc * C, nc = min(C, T - t0c);
    constexpr int PPK = DK / 8;  // 16-byte pieces per q or k row
    const int64_t e0 = (tok0 + t0c) * H * DK + (int64_t)h * DK;
    const uint32_t bytes = (uint32_t)(nc - 1) * rowq + DK * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + e0, bytes);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + e0, bytes);
    const int ln = opaque(lane);
    for (int j = wv; j * 64 < C * PPK; j += nw) {
      const int p = j * 64 + ln, r = p / PPK, pc = p % PPK;
      const uint32_t off = (uint32_t)r * rowq + (uint32_t)pc * 16;
      if (p < C * PPK && r < nc) {
        dma_buf<16>(rk, off, lKr + j * 1024);
        if (OUTM) dma_buf<16>(rq, off, lQr + j * 1024);
      }
    }
  };
  // the gate rows of chunk cc (one wave), into raw gate buffer cc & 1
  auto issue_g = [&](int cc) {
    const int t0c = cc * C, nc = min(C, T - t0c);
    const int ln = opaque(lane);
    lds_char* dst = lGr + (cc & 1) * (C * 6 * 4);
    if (ln < nc) {
      const int64_t gidx = (tok0 + t0c) * H + h;
      const uint32_t gb = (uint32_t)(nc - 1) * H * 4 + 4;
      const uint32_t off = (uint32_t)(ln * H) * 4;
      dma_buf<4>(make_rsrc(a.alpha + gidx, gb), off, dst);
      dma_buf<4>(make_rsrc(a.beta + gidx, gb), off, dst + C * 4);
      dma_buf<16>(make_rsrc(a.taps + gidx * 4, gb * 4), off * 4, dst + 2 * C * 4);
    }
  };
  // gates of chunk cc (wave GW, its raw gate rows in LDS): the cumulative log
  // decay g (base 2), gamma = 2^g, beta and e^{g_C - g} into gate buffer cc & 1,
  // and the chunk's band coefficients
  auto gates = [&](int cc) {
    const int nc = min(C, T - cc * C);
    const float* gr = sGr + (cc & 1) * (C * 6);
    float* gg = sG2 + (cc & 1) * (4 * C);
    const bool valid = lane < nc;
    const float al = valid ? gr[lane] : 1.f;
    const float be = valid ? gr[C + lane] : 0.f;
    const float4 tp = valid ? reinterpret_cast<const float4*>(gr + 2 * C)[lane] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float g = chunk_gate_scan(al);
    const float gC = __shfl(g, C - 1, WAVE);
    gg[lane] = g;
    gg[C + lane] = fast_exp2(g);
    gg[2 * C + lane] = be;
    gg[3 * C + lane] = fast_exp2(gC - g);
    // row `lane` of the band with Band[r][r + j] = b_r tap_r[j], so that
    // diag(b) V' = Band V_ext runs on the matrix cores: row tile rt takes the
    // 32 staged value rows from 16 rt (from C + 3 - 32 for the last tile),
    // each coefficient split into bf16 hi + lo
    const int rt = lane >> 4, m = lane & 15, k0 = (rt < 3 ? 0 : 16 * rt - (C + 3 - 32)) + m;
    const float cf[4] = {be * tp.x, be * tp.y, be * tp.z, be * tp.w};
    // (one opaque offset: the address stays a short chain from the LDS array,
    // so the compiler can tell these stores from the DMA's)
    const int to = opaque((rt * 16 + m) * LT + k0);
    bf16_t* th = sT + to;
    bf16_t* tl = sT + (to + 4 * 16 * LT);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16_t hi = f32_to_bf16(cf[j]);
      th[j] = hi;
      tl[j] = f32_to_bf16(cf[j] - bf16_to_f32(hi));
    }
  };
  // value rows (with the conv halo) of chunk cc, shared by waves w0 .. w0 + nw - 1.
  // Row r holds token t0c - 3 + r.  Past the sequence's first chunk all rows
  // come from v: one full-wave DMA per 1 KB group of rows (wave w takes groups
  // w - w0, w - w0 + nw, ..), rows past the sequence end reading zero through
  // the buffer range.  In the first chunk the halo rows come from
  // the conv cache (or are zero): one DMA per row.
  auto issue_v = [&](int cc, int w0, int nw) {
    const int t0c = cc * C, nc = min(C, T - t0c);
    constexpr int PPR = DV / 8;  // 16-byte pieces per value row
    // rows from token rb0 (the halo's first row, or the chunk's when it starts the sequence)
    const int rb0 = t0c >= 3 ? t0c - 3 : t0c;
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(v + ((tok0 + rb0) * H + h) * DV, (uint32_t)(t0c + nc - 1 - rb0) * rowv + DV * 2);
    const int ln = opaque(lane);
    if (t0c >= 3) {
      // lane ln fills slot ln % PPR of row ln / PPR of the group
      const int j = ln / PPR;
      const uint32_t lo = (uint32_t)j * rowv + (uint32_t)((ln % PPR) ^ (2 * G::vsw(j))) * 16;
      for (int g = wave - w0; g < NVG; g += nw)
        dma_buf<16>(rv, (uint32_t)(g * VRPG) * rowv + lo, lVw + g * VG);
      return;
    }
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(cin ? cin + ((int64_t)b * 3 * H + h) * DV : v, cin ? 2 * rowv + DV * 2 : 0u);

    for (int r = wave - w0; r < C + 3; r += nw) {
      const int t = t0c - 3 + r;
      lds_char* dst = lVw + G::vrow(r);
      const uint32_t pc = (uint32_t)(ln ^ (2 * G::vsw(r % VRPG))) * 16;  // piece for slot ln
      if (ln < PPR) {
        if (t >= 0 && r - 3 < nc)
          dma_buf<16>(rv, (uint32_t)(t - rb0) * rowv + pc, dst);
        else if (t < 0 && cin)
          dma_buf<16>(rc, (uint32_t)(3 + t) * rowv + pc, dst);
        else
          *(__attribute__((address_space(3))) u4_t*)(dst + ln * 16) = u4_t{0u, 0u, 0u, 0u};
      }
    }
  };

  // a column tile of outputs, rows t0 .. t0 + n - 1, straight from registers:
  // the tile is held transposed (lane 16 g + m has row m of each 16-row block,
  // columns 4 g .. 4 g + 3), so every lane stores four adjacent outputs at once
  auto store_o = [&](const f4_t (&Ot)[4], int ct, int t0, int n, int E) {
    const uint32_t rowb = (uint32_t)(H * DV * (int)sizeof(OUT));
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(reinterpret_cast<OUT*>(a.o) + ((tok0 + t0) * H + h) * DV, (uint32_t)n * rowb);
    const int ovoff = (int)(m16 * rowb) + (ct * 16 + 4 * g4) * (int)sizeof(OUT);
    const int e = held_exp(E);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const float x0 = ldexpf(Ot[rt][0], e), x1 = ldexpf(Ot[rt][1], e);
      const float x2 = ldexpf(Ot[rt][2], e), x3 = ldexpf(Ot[rt][3], e);
      // rows at or beyond n fall outside the resource and are dropped
      if constexpr (sizeof(OUT) == 2) {
        const uint32_t w0 = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16(x2) | ((uint32_t)f32_to_bf16(x3) << 16);
        __builtin_amdgcn_raw_buffer_store_b64(u2_t{w0, w1}, orsrc, ovoff, (int)(rt * 16 * rowb), 0);
      } else {
        // two 8-byte stores: a wider store's data registers may still be read
        // after the next instruction has overwritten them (the compiler does not
        // guard that case when the offset is in an SGPR)
        __builtin_amdgcn_raw_buffer_store_b64(u2_t{__float_as_uint(x0), __float_as_uint(x1)}, orsrc, ovoff,
                                              (int)(rt * 16 * rowb), 0);
        __builtin_amdgcn_raw_buffer_store_b64(u2_t{__float_as_uint(x2), __float_as_uint(x3)}, orsrc, ovoff + 8,
                                              (int)(rt * 16 * rowb), 0);
      }
    }
  };

  // bf16 o rows of a chunk in LDS: row r at r * DV * 2 bytes, its 16-byte
  // pieces permuted by the row (piece p sits at p ^ (r % (DV / 8))) so that the
  // tile writes below (16 rows, one 16-byte piece each per half wave) touch
  // every bank once
  lds_char* lSO = (lds_char*)work + G::oSO;
  auto so_addr = [&](int row, int cbyte) {  // cbyte: byte offset in the row
    return row * (DV * 2) + (cbyte ^ ((row & (DV / 8 - 1)) << 4));
  };
  // a column tile of outputs (held transposed, as in store_o) into the staging rows
  auto stage_o = [&](const f4_t (&Ot)[4], int ct, int E) {
    const int e = held_exp(E);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const uint32_t w0 = (uint32_t)f32_to_bf16(ldexpf(Ot[rt][0], e)) |
                          ((uint32_t)f32_to_bf16(ldexpf(Ot[rt][1], e)) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(ldexpf(Ot[rt][2], e)) |
                          ((uint32_t)f32_to_bf16(ldexpf(Ot[rt][3], e)) << 16);
      *(__attribute__((address_space(3))) u2_t*)(lSO + opaque(so_addr(rt * 16 + m16, ct * 32 + 8 * g4))) =
          u2_t{w0, w1};
    }
  };
  // the staged rows t0p .. t0p + np - 1 to o: whole rows, 16 bytes per lane
  // (rows at or beyond np fall outside the resource and are dropped)
  auto flush_o = [&](int t0p, int np) {
    constexpr int LPR = DV * 2 / 16;  // lanes per row
    constexpr int RPI = 64 / LPR;     // rows per store
    const uint32_t rowb = (uint32_t)(H * DV * 2);
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(reinterpret_cast<OUT*>(a.o) + ((tok0 + t0p) * H + h) * DV, (uint32_t)np * rowb);
    const int ln = opaque(lane);
    const int cb = (ln % LPR) * 16;
#pragma unroll
    for (int i = 0; i < C / (NW * RPI); ++i) {
      const int row = (wave * (C / (NW * RPI)) + i) * RPI + ln / LPR;
      const u4_t val = *(const __attribute__((address_space(3))) u4_t*)(lSO + so_addr(row, cb));
      // a zero soffset: the compiler then guards the store's data registers
      __builtin_amdgcn_raw_buffer_store_b128(val, orsrc, (int)(row * rowb) + cb, 0, 0);
    }
  };
  int pend_t0 = 0, pend_n = 0;

  if (c_begin < c_end) {
    issue_qkg(c_begin, wave, NW);
    issue_v(c_begin, 0, NW);
    // the gate rows run two chunks ahead (those of chunk c + 2 move during
    // chunk c; chunk c + 1's gates are formed in chunk c's phase D)
    if (wave == G::GW) {
      issue_g(c_begin);
      if (c_begin + 1 < c_end) issue_g(c_begin + 1);
    }
    // the first chunk's rows land before the loop, so that at the top of every
    // iteration the transfers still outstanding are those the previous chunk
    // issued, followed by its o stores
    __builtin_amdgcn_s_waitcnt(0);
    if (wave == G::GW) gates(c_begin);
  }
  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * C;
    const int n = min(C, T - t0);
    const float* sG = sG2 + (c & 1) * (4 * C);
    const float* sGam = sG + C;
    const float* sBeta = sG + 2 * C;
    const float* sDec = sG + 3 * C;
    // this wave's DMA transfers into the staging areas are done, then every
    // other wave's.  (The wait covers the previous chunk's o stores as well:
    // loads and stores share the vector memory counter and need not complete
    // in order with respect to each other, so no count short of zero proves
    // the transfers done.)
    __builtin_amdgcn_s_waitcnt(0);
    bar();

    // the previous chunk's outputs, staged in LDS, leave first (their region is
    // next written in phase B)
    if constexpr (STAGE_O)
      if (c > c_begin) flush_o(pend_t0, pend_n);

    // ================= A: normalise q, k; gates and band =================
    {
      constexpr int E = DK / 8;
      const int row = tid >> 3, part = tid & 7;
      const bool valid = row < n;
      float kv[E];
      load_row_part<bf16_t>(sKr + row * DK + part * E, kv, E, valid);
      float sk = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) sk += kv[e] * kv[e];
      const float rk = l2_scale(group_sum<8>(sk));
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const h2_t x0 = __builtin_convertvector(f2_t{kv[e] * rk, kv[e + 1] * rk}, h2_t);
        const h2_t x1 = __builtin_convertvector(f2_t{kv[e + 2] * rk, kv[e + 3] * rk}, h2_t);
        *reinterpret_cast<h4_t*>(sKh + row * LDK + part * E + e) = h4_t{x0[0], x0[1], x1[0], x1[1]};
      }
      if (OUTM) {
        float qv[E];
        load_row_part<bf16_t>(sQr + row * DK + part * E, qv, E, valid);
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) sq += qv[e] * qv[e];
        const float rq = l2_scale(group_sum<8>(sq));
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          const h2_t x0 = __builtin_convertvector(f2_t{qv[e] * rq, qv[e + 1] * rq}, h2_t);
          const h2_t x1 = __builtin_convertvector(f2_t{qv[e + 2] * rq, qv[e + 3] * rq}, h2_t);
          *reinterpret_cast<h4_t*>(sQh + row * LDK + part * E + e) = h4_t{x0[0], x0[1], x1[0], x1[1]};
        }
      }
    }
    bar();

    // ================= B: Gram tiles and diagonal inverses; right-hand sides,
    // tile exponents, Q^ M =================
    // Gram tile (ti, tj), formed transposed: lane holds (Y K^T)[16 ti + m16][16 tj + 4 g4 + i]
    // (Y = K^ or Q^), so -A, P and the diagonal blocks are written as whole rows
    auto gram = [&](int ti, int tj) {
      f4_t kk = zero4(), qk = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const half8_t ak = row_frag_ct<LDK>(rKct, tj * 16, kb * 32);
        kk = mfma(ak, row_frag_ct<LDK>(rKct, ti * 16, kb * 32), kk);
        if (OUTM) qk = mfma(ak, row_frag_ct<LDK>(rQct, ti * 16, kb * 32), qk);
      }
      const int ln = opaque(lane);
      const int r = ti * 16 + (ln & 15), c0 = tj * 16 + 4 * (ln >> 4);
      const float gr = sG[r], br = sBeta[r];
      const float4 gc = *reinterpret_cast<const float4*>(sG + c0);
      const float gcv[4] = {gc.x, gc.y, gc.z, gc.w};
      float an[4], pp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float E = fast_exp2(gr - gcv[i]);
        const int cc = c0 + i;
        an[i] = cc < r ? br * E * kk[i] : 0.f;
        pp[i] = cc <= r ? E * qk[i] : 0.f;
      }
      const h2_t a0 = __builtin_convertvector(f2_t{-an[0], -an[1]}, h2_t);
      const h2_t a1 = __builtin_convertvector(f2_t{-an[2], -an[3]}, h2_t);
      *reinterpret_cast<h4_t*>(sAn + r * LC + c0) = h4_t{a0[0], a0[1], a1[0], a1[1]};
      if (ti == tj) *reinterpret_cast<float4*>(sAd + r * LAD + c0 - tj * 16) = make_float4(an[0], an[1], an[2], an[3]);
      if (OUTM) {
        const h2_t p0 = __builtin_convertvector(f2_t{pp[0], pp[1]}, h2_t);
        const h2_t p1 = __builtin_convertvector(f2_t{pp[2], pp[3]}, h2_t);
        *reinterpret_cast<h4_t*>(sP + r * LC + c0) = h4_t{p0[0], p0[1], p1[0], p1[1]};
      }
    };
    if (wave >= 4) {
      // diagonal tile d = wave - 4, then the inverse of I + A's diagonal block d
      // by forward substitution (column jc = lane % 16; lanes 16.. repeat lanes 0..15)
      const int d = wave - 4;
      gram(d, d);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's block rows are in LDS
      const int base = d * 16;
      int jc = lane & 15;
      asm volatile("" : "+v"(jc));  // formed per chunk: the 16 identity values are not held across the loop
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
      if (lane < 16) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sLi[(base + i) * LLI + jc] = (_Float16)x[i];
          sLi[(base + i) * LLI + 16 + jc] = (_Float16)0.f;  // the zero half a 32-deep fragment reads
        }
      }
    } else {
      // off-diagonal tiles (1,0) (2,0) (2,1) (3,0) (3,1) (3,2): jobs wave and wave + 4
      constexpr uint32_t kOffI = 0xfe9u, kOffJ = 0x910u;  // two bits per job
      gram((kOffI >> (2 * wave)) & 3, (kOffJ >> (2 * wave)) & 3);
      if (wave < 2) gram((kOffI >> (2 * wave + 8)) & 3, (kOffJ >> (2 * wave + 8)) & 3);
      // these waves are done with the Gram work first: they move the next
      // chunk's q, k and gate rows (the staging areas were last read in phase A)
      if (c + 1 < c_end) issue_qkg(c + 1, wave, 4);
      if (wave == 3 && c + 2 < c_end) issue_g(c + 2);
      if constexpr (STAGE_O) {
        // the two zero blocks above P's block diagonal that P V_new reads,
        // rows 0..15 x columns 16..31 and rows 32..47 x columns 48..63 (the
        // o staging rows of the previous chunk lay over them)
        if (wave == 3) {
          const int blk = lane >> 5, r = blk * 32 + ((lane & 31) >> 1), c0 = blk * 32 + 16 + 8 * (lane & 1);
          *reinterpret_cast<u4_t*>(sP + opaque(r * LC + c0)) = u4_t{0u, 0u, 0u, 0u};
        }
      }
    }
    // the rest of the phase after the Gram work (waves 0..3 and 4..7 share the
    // SIMDs pairwise, so the other wave fills a SIMD while one inverts)
    __builtin_amdgcn_sched_barrier(0);
    f4_t U[TPW][4];
#pragma unroll
    for (int cw = 0; cw < TPW; ++cw) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) U[cw][rt] = zero4();
      if (!isval(cw)) continue;
      // right-hand side diag(b) V': tile rt = (Band_hi + Band_lo) V_ext[window rows][column tile],
      // the value rows taken exactly as bf16 operands (kperm K order on both sides)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const bf16x8_t th = __builtin_bit_cast(bf16x8_t, row_frag_kp<LT>(rTkp, rt * 16, 0));
        const bf16x8_t tl = __builtin_bit_cast(bf16x8_t, row_frag_kp<LT>(rTkp, (4 + rt) * 16, 0));
        // window rows 16 rt .. (rt < 3) or C + 3 - 32 .. (the last): two 16-row halves
        const lds_char* vbase = rt < 3 ? tVa + G::vrow(16 * rt) : tVb;
        const s4_t vlo = tr4(vbase + cw * NW * 32);
        const s4_t vhi = tr4(vbase + (16 / VRPG) * VG + cw * NW * 32);
        const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7));
        const f4_t hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th, vb, zero4(), 0, 0, 0);
        U[cw][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl, vb, hi, 0, 0, 0);
      }
    }
#pragma unroll
    for (int cw = 0; cw < TPW; ++cw)
      if (has(cw)) rescale_tile(Macc[cw], U[cw], Ex[cw]);
    // R = diag(b) V' - diag(b gamma) K^ M (both now at the tile's scale): the rows
    // of K^ scaled by -b gamma of their token (the A fragment's row is the
    // lane's), onto the band product; with the same fragments of M, the output
    // pass forms Q^ M (transposed, as the o tiles are held)
    f4_t O[OUTM ? TPW : 1][4];
    if constexpr (OUTM) {
#pragma unroll
      for (int cw = 0; cw < TPW; ++cw)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) O[cw][rt] = zero4();
    }
    {
      _Float16 bg[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) bg[rt] = (_Float16)(-sBeta[rt * 16 + m16] * sGam[rt * 16 + m16]);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        half8_t mk[TPW];  // this chunk's M as fp16 fragments (kperm rows)
#pragma unroll
        for (int cw = 0; cw < TPW; ++cw) mk[cw] = acc_frag2(Macc[cw][2 * kb], Macc[cw][2 * kb + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const half8_t ak = row_frag_kp<LDK>(rKkp, rt * 16, kb * 32) * bg[rt];
#pragma unroll
          for (int cw = 0; cw < TPW; ++cw)
            if (has(cw)) U[cw][rt] = mfma(ak, mk[cw], U[cw][rt]);
          if constexpr (OUTM) {
            const half8_t aq = row_frag_kp<LDK>(rQkp, rt * 16, kb * 32);
#pragma unroll
            for (int cw = 0; cw < TPW; ++cw)
              if (has(cw)) O[cw][rt] = mfma(mk[cw], aq, O[cw][rt]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // one K block of fragments in registers at a time
      }
    }
    if constexpr (OUTM) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float gm = sGam[rt * 16 + m16];  // the row of O this lane holds
#pragma unroll
        for (int cw = 0; cw < TPW; ++cw)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[cw][rt][i] *= gm;
      }
    }
    bar();
    // the next chunk's value rows (every wave is past its band product), moved
    // by the waves that wait out the solve (the DMA issue stalls a wave while
    // the CU's load path is busy)
    if (c + 1 < c_end && wave >= 4 && wave < G::GW) issue_v(c + 1, 4, G::GW - 4);

    // ================= D: T = (I + A)^{-1} by blocked forward substitution,
    // column block j on wave j (its columns of the identity as right-hand side)
    if (wave < 4) {
      const int j = wave, jm = opaque(m16 - 4 * g4);  // lane's identity entry: row 16 j + 4 g4 + i == 16 j + m16
      f4_t Y[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[rb][i] = (rb == j && i == jm) ? 1.f : 0.f;
      solve<LC, LLI>(Y, rAkp, rLkp);
      // T^T: row 16 j + m16, columns 16 rb + 4 g4 .. + 3 (zero above the diagonal blocks)
      _Float16* sTt = reinterpret_cast<_Float16*>(work + G::oQW);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const h2_t w0 = __builtin_convertvector(f2_t{Y[rb][0], Y[rb][1]}, h2_t);
        const h2_t w1 = __builtin_convertvector(f2_t{Y[rb][2], Y[rb][3]}, h2_t);
        *reinterpret_cast<h4_t*>(sTt + opaque((j * 16 + m16) * LTT + rb * 16 + 4 * g4)) =
            h4_t{w0[0], w0[1], w1[0], w1[1]};
      }
    } else if (wave == G::GW && c + 1 < c_end) {
      // the next chunk's gates (its raw rows landed by this chunk's top wait;
      // the band was last read in phase B, the gate buffer in the previous chunk)
      gates(c + 1);
    }
    bar();

    // ================= E: state-dependent part of the chunk =================
    // V_new = T R (T read down the columns of T^T; row block rt takes K blocks
    // kb <= rt / 2, T being lower triangular), over R in place
    {
      half8_t rf[TPW][2];
#pragma unroll
      for (int cw = 0; cw < TPW; ++cw)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) rf[cw][kb] = acc_frag2(U[cw][2 * kb], U[cw][2 * kb + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const half8_t t0f = tr_frag_kp<LTT>(tTkp, 0, rt * 16);
#pragma unroll
        for (int cw = 0; cw < TPW; ++cw)
          if (has(cw)) U[cw][rt] = mfma(t0f, rf[cw][0], zero4());
        if (rt >= 2) {
          const half8_t t1f = tr_frag_kp<LTT>(tTkp, 32, rt * 16);
#pragma unroll
          for (int cw = 0; cw < TPW; ++cw)
            if (has(cw)) U[cw][rt] = mfma(t1f, rf[cw][1], U[cw][rt]);
        }
      }
    }
    if constexpr (OUTM) {
      // O += P V_new, then the outputs
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        half8_t vn[TPW];
#pragma unroll
        for (int cw = 0; cw < TPW; ++cw) vn[cw] = acc_frag2(U[cw][2 * kb], U[cw][2 * kb + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          if (kb * 32 <= rt * 16 + 15) {
            const half8_t ap = row_frag_kp<LC>(rPkp, rt * 16, kb * 32);
#pragma unroll
            for (int cw = 0; cw < TPW; ++cw)
              if (has(cw)) O[cw][rt] = mfma(vn[cw], ap, O[cw][rt]);
          }
        __builtin_amdgcn_sched_barrier(0);  // one K block of fragments in registers at a time
      }
      if constexpr (STAGE_O) {
        bar();  // every wave is done with P (and -A, its diagonal blocks and their inverses)
#pragma unroll
        for (int cw = 0; cw < TPW; ++cw)
          if (has(cw)) stage_o(O[cw], tile(cw), Ex[cw]);
        pend_t0 = t0;  // stored at the start of the next chunk
        pend_n = n;
      } else {
#pragma unroll
        for (int cw = 0; cw < TPW; ++cw)
          if (has(cw)) store_o(O[cw], tile(cw), t0, n, Ex[cw]);
      }
    }
    // M <- gamma_C M + K^T diag(e^{g_C - g}) V_new (K^ read down its columns)
    {
      const float gamC = sGam[C - 1];
#pragma unroll
      for (int cw = 0; cw < TPW; ++cw)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) Macc[cw][rt][i] *= gamC;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 d0 = *reinterpret_cast<const float4*>(sDec + kb * 32 + 4 * g4);
        const float4 d1 = *reinterpret_cast<const float4*>(sDec + kb * 32 + 16 + 4 * g4);
        half8_t vd[TPW];
#pragma unroll
        for (int cw = 0; cw < TPW; ++cw) vd[cw] = acc_frag2_scaled(U[cw][2 * kb], U[cw][2 * kb + 1], d0, d1);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const half8_t ak = tr_frag_kp<LDK>(tKkp, kb * 32, rt * 16);
#pragma unroll
          for (int cw = 0; cw < TPW; ++cw)
            if (has(cw)) Macc[cw][rt] = mfma(ak, vd[cw], Macc[cw][rt]);
        }
        __builtin_amdgcn_sched_barrier(0);  // one K block of fragments in registers at a time
      }
    }
  }

  if constexpr (STAGE_O) {
    if (c_begin < c_end) {
      bar();
      flush_o(pend_t0, pend_n);
    }
  }

  // ---- results (true units)
#pragma unroll
  for (int cw = 0; cw < TPW; ++cw) {
    if (!has(cw)) continue;
    const int ct = tile(cw);
    const int e = held_exp(Ex[cw]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + 4 * g4 + i;
        const float mv = ldexpf(Macc[cw][rt][i], e);
        if (OUTM) {
          if (s == nseg_b - 1) a.S_final[(bh * DK + row) * DV + ct * 16 + m16] = mv;
        } else if (ct < VCT) {
          a.Dsum[((bh * a.nseg + s) * DK + row) * DV + ct * 16 + m16] = mv;
        } else {
          a.Phi[((bh * a.nseg + s) * DK + row) * DK + (ct - VCT) * 16 + m16] = mv;
        }
      }
  }
}

}  // namespace fwd

// ------------------------------------------------------------ host side

#define JB_FWD_CASES(X) \
  X(32, 64) X(32, 128) X(32, 256) X(64, 64) X(64, 128) X(64, 256) \
  X(96, 64) X(96, 128) X(96, 256) X(128, 64) X(128, 128) X(128, 256)

bool fwd_supported(int dk, int dv) {
#define CASE(DK_, DV_) if (dk == DK_ && dv == DV_) return true;
  JB_FWD_CASES(CASE)
#undef CASE
  return false;
}

template <int DK, int DV, typename OUT>
static hipError_t run_fwd(const FwdArgs& a, int passes, int nseg, int H, int B, hipStream_t stream) {
  using GS = fwd::Geo<DK, DV, fwd::SUMMARY>;
  using GO = fwd::Geo<DK, DV, fwd::OUTPUT>;
  if (passes & 1)
    fwd::fwd_kernel<DK, DV, OUT, fwd::SUMMARY><<<dim3(nseg - 1, H, B), dim3(GS::NW * 64), 0, stream>>>(a);
  if (passes & 2)
    fwd::fwd_kernel<DK, DV, OUT, fwd::OUTPUT><<<dim3(nseg, H, B), dim3(GO::NW * 64), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int passes, int dk, int dv, bool out_bf16, int nseg, int H, int B,
                      hipStream_t stream) {
#define CASE(DK_, DV_)                                                                  \
  if (dk == DK_ && dv == DV_)                                                           \
    return out_bf16 ? run_fwd<DK_, DV_, bf16_t>(a, passes, nseg, H, B, stream)          \
                    : run_fwd<DK_, DV_, float>(a, passes, nseg, H, B, stream);
  JB_FWD_CASES(CASE)
#undef CASE
  return hipErrorInvalidValue;
}

}  // namespace jb
