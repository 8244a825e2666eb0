// jb_proj.hip -- the block's input projections (q, k, v, the gates) and the
// kernel generator from one pass over x.
//
// The kernel generator takes the same input as the Q/K/V projection layers
// (Jet-Nemotron csdn translation, section 2.4), so the block can start from
// the layer input x instead of from q, k, v:
//     q = Wq x,  k = Wk x,  v = Wv x                          (bf16 out)
//     alpha = sigmoid(Wa x + ba),  beta = sigmoid(Wb x + bb)  (one per head)
//     taps  = W2 SiLU(W1 x + b1) + b2                          (4 per head)
// The gate projections are not described on the pages; a sigmoid keeps both
// gates in (0, 1) as the recurrence needs.
//
// One kernel forms all of it.  The output features are laid end to end:
// [q: H dk | k: H dk | v: H dv] in tiles of BF features, then (when W1 is
// given) one more tile holding [W1: 32 | Wa: H | Wb: H] (Wa and Wb each
// padded to a multiple of 16 rows).  A workgroup computes
// one BT-token x BF-feature tile as the transposed product
// Y^T = W x^T on bf16 matrix cores with fp32 accumulation, so that every lane
// ends holding four consecutive features of one token: q, k and v are
// rounded once to bf16 and stored, and the generator tile applies SiLU, the
// 32 -> 4H second layer and the gate sigmoids in fp32 before its stores.
//
// The K loop streams 32-deep slices of x and W rows into LDS with direct
// buffer -> LDS loads (16 bytes per lane), NST slices in flight.  Within a row of a slice the 16-byte pieces are permuted
// by a function of the row so that the fragment reads (16 rows, same piece)
// hit distinct banks.  Tiles are numbered so that each of the chip's eight
// dies (blocks go round-robin over them) gets a contiguous run, ordered in
// groups of GM token tiles with the feature tiles outside, so the x rows and
// W rows the resident workgroups share stay in the die's L2.
#include "jb_device.h"
#include "jb_internal.h"

namespace jb {

namespace {

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;

constexpr int GH = 32;  // generator hidden width

struct ProjArgs {
  const bf16_t* x;
  int64_t n;                 // tokens
  int D, H, Nq, Nv;          // Nq = H dk, Nv = H dv
  const bf16_t *Wq, *Wk, *Wv, *W1, *Wa, *Wb;
  const bf16_t *b1, *W2, *b2, *ba, *bb;
  bf16_t *q, *k, *v;
  float *alpha, *beta, *taps;
  int nft;                   // feature tiles over q, k, v
  int ntf;                   // feature tiles in all (nft, + 1 for the generator tile)
  int mtiles;                // token tiles
};

__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// barrier after this wave's LDS accesses have completed
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A raw buffer descriptor over [base, base + bytes): reads past the range
// return zero.  Wave-uniform by construction; readfirstlane says so to the
// register allocator, which then keeps it in scalar registers.
typedef int v4i_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i_t buf_desc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return v4i_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
               __builtin_amdgcn_readfirstlane((int)(uint32_t)((b >> 32) & 0xffff)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// Buffer -> LDS load of 16 bytes per lane: the piece at byte voff + soff of the
// buffer lands at LDS byte lds + 16 lane.  Written out so that the compiler
// does not track it: it would otherwise wait for every such load in flight
// before each LDS read of the K loop.  The loop's own s_waitcnt on the
// vector-memory count and its barriers order the slices.  The load has no
// register result, only the LDS bytes it writes; M0 (the LDS base, read when
// the load issues) is restored afterwards.
// The leading s_nop covers a vector-ALU write (readfirstlane) of the
// descriptor or offsets just before, which the compiler cannot see here.
__device__ __forceinline__ void dma16(v4i_t desc, int voff, int soff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_nop 4\n\ts_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(desc), "s"(soff), "s"(lds)
      : "memory");
}

// slot of 16-byte piece p in LDS row r: p ^ swz(r), with swz a function of
// r mod 16 (the same for every 16-row block a lane reads).  Chosen by
// measurement (SQ_LDS_BANK_CONFLICT on the fragment reads: 16 rows, one
// piece per lane group): r mod 8 for 128-byte rows and (r/2 ^ r/4) mod 4 for
// 64-byte rows leave about 1% of LDS cycles in conflicts, where
// (r mod 8) ^ (r/8 mod 2) leaves 49% and no permutation 74%.
template <int BK>
__device__ __forceinline__ int swz(int r) {
  if constexpr (BK == 64) return r & 7;
  else return ((r >> 1) ^ (r >> 2)) & 3;
}

template <int BT_, int BF_, int WT_, int WF_, int BK_, int NST_, int GM_, int MINW_>
struct Cfg {
  static constexpr int BT = BT_, BF = BF_, WT = WT_, WF = WF_, BK = BK_, NST = NST_, GM = GM_, MINW = MINW_;
  static constexpr int NWT = BT / WT, NWF = BF / WF, NW = NWT * NWF, NTHR = NW * 64;
  static constexpr int ROWB = BK * 2;              // bytes per LDS row
  static constexpr int PPR = BK / 8;               // 16-byte pieces per row
  static constexpr int RPI = 64 / PPR;             // rows per load instruction
  static constexpr int STAGE = (BF + BT) * ROWB;   // bytes per slice: BF W rows, then BT x rows
  static constexpr int NDMA = (BF + BT) / RPI;
  static constexpr int DPW = NDMA / NW;            // load instructions per wave and slice
  static constexpr int FI = WF / 16, TJ = WT / 16, KK = BK / 32;
  static constexpr int RING = NST * STAGE;
  static_assert(NDMA % NW == 0 && BF % RPI == 0, "slice loads split evenly over the waves");
  static_assert(64 % WT == 0 || WT % 64 == 0, "token passes of the generator epilogue");
  static_assert((NST & (NST - 1)) == 0 && NST >= 2, "a power-of-two ring of slices");
  static_assert((NST - 2) * DPW < 64, "loads in flight fit the vector-memory counter");
  static_assert(RING >= (64 + 128) * (32 + 1) * 4, "the generator epilogue reuses the ring");
  static_assert(BK == 32 || BK == 64, "slice depth");
};

// Wait until at most min(ahead, M) slices of DPW loads each are still in flight.
template <int DPW, int M>
__device__ __forceinline__ void wait_slices(int ahead) {
  if constexpr (M <= 0) {
    wait_vm<0>();
  } else {
    if (ahead >= M) wait_vm<M * DPW>();
    else wait_slices<DPW, M - 1>(ahead);
  }
}

// Which (token tile, feature tile) block g computes.
template <class C>
__device__ __forceinline__ void tile_of(int64_t g, const ProjArgs& a, int& mb, int& ft) {
  const int64_t total = (int64_t)a.mtiles * a.ntf;
  const int64_t per = total / 8, rem = total % 8;
  const int64_t x = g % 8, i = g / 8;
  const int64_t L = x * per + (x < rem ? x : rem) + i;
  const int64_t grp = L / ((int64_t)C::GM * a.ntf), w = L % ((int64_t)C::GM * a.ntf);
  const int64_t left = (int64_t)a.mtiles - grp * C::GM;
  const int gm = (int)(left < C::GM ? left : C::GM);
  ft = (int)(w / gm);
  mb = (int)(grp * C::GM + w % gm);
}

// The W rows feeding LDS rows [R0, R0 + 16) of a feature tile: a 16-row run
// never straddles two matrices (H dk and H dv are multiples of 32; in the
// generator tile the Wa and Wb rows start on 16-row boundaries: features
// [W1: 32 | Wa: H, padded to P | Wb: H, padded]).  Rows past a matrix's end
// read as zero through the buffer range.
struct RowRun {
  const bf16_t* base;
  int row0, rows;
};
__device__ __forceinline__ RowRun w_run(const ProjArgs& a, bool gen, int F0) {
  if (!gen) {
    if (F0 < a.Nq) return {a.Wq, F0, a.Nq};
    if (F0 < 2 * a.Nq) return {a.Wk, F0 - a.Nq, a.Nq};
    if (F0 < 2 * a.Nq + a.Nv) return {a.Wv, F0 - 2 * a.Nq, a.Nv};
    return {a.Wv, a.Nv, a.Nv};
  }
  const int P = (a.H + 15) & ~15;
  if (F0 < GH) return {a.W1, F0, GH};
  if (F0 < GH + P) return {a.Wa, F0 - GH, a.H};
  if (F0 < GH + 2 * P) return {a.Wb, F0 - GH - P, a.H};
  return {a.W1, GH, GH};
}

template <class C>
__global__ __launch_bounds__(C::NTHR, C::MINW) void proj_kernel(ProjArgs a) {
  // NST slices of the K loop; after it, the generator tile's hidden layer and W2
  __shared__ __attribute__((aligned(16))) char ring[C::RING];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: buffer ranges stay scalar
  const int m16 = lane & 15, g4 = lane >> 4;
  const int wt = wave % C::NWT, wf = wave / C::NWT;
  int mb, ft;
  tile_of<C>(blockIdx.x, a, mb, ft);
  const int64_t t0 = (int64_t)mb * C::BT;
  const bool gen = ft >= a.nft;
  const int f0 = gen ? 0 : ft * C::BF;
  const int64_t D = a.D;

  // this lane's piece of each of its load instructions: a buffer range per
  // instruction (wave-uniform) and a byte offset per lane; slice kt adds kt ROWB
  v4i_t rsrc[C::DPW];
  int voff[C::DPW];
#pragma unroll
  for (int i = 0; i < C::DPW; ++i) {
    const int j = wave + C::NW * i;
    const int R0 = j * C::RPI, R = R0 + lane / C::PPR;
    const int piece = (lane % C::PPR) ^ swz<C::BK>(R);
    if (R0 < C::BF) {
      const RowRun w = w_run(a, gen, f0 + R0);
      rsrc[i] = buf_desc(w.base, (uint32_t)((int64_t)w.rows * D * 2));
      voff[i] = ((w.row0 + lane / C::PPR) * a.D + piece * 8) * 2;
    } else {
      const int64_t left = a.n - t0;
      rsrc[i] = buf_desc(a.x + t0 * D, (uint32_t)((left < C::BT ? left : C::BT) * D * 2));
      voff[i] = ((R - C::BF) * a.D + piece * 8) * 2;
    }
  }
  lds_char* const R0 = (lds_char*)ring;
  auto issue = [&](int kt) {
    lds_char* S = R0 + (kt & (C::NST - 1)) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::DPW; ++i) {
      const int j = wave + C::NW * i;
      dma16(rsrc[i], voff[i], kt * C::ROWB, (uint32_t)(uintptr_t)(S + j * 1024));
    }
  };

  // fragment reads: lane row m16 of each 16-row block, piece 4 kk + g4 (K 32 kk + 8 g4 .. + 7)
  const int ra = wf * C::WF + m16, rb = C::BF + wt * C::WT + m16;
  int aoff[C::KK], boff[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk) {
    aoff[kk] = ra * C::ROWB + (((4 * kk + g4) ^ swz<C::BK>(ra)) * 16);
    boff[kk] = rb * C::ROWB + (((4 * kk + g4) ^ swz<C::BK>(rb)) * 16);
  }
  // a wave of the generator tile whose features are all past the gates has nothing to compute
  const int P = (a.H + 15) & ~15;
  const bool live = !gen || wf * C::WF < GH + 2 * P;

  f4_t acc[C::FI][C::TJ];
#pragma unroll
  for (int i = 0; i < C::FI; ++i)
#pragma unroll
    for (int j = 0; j < C::TJ; ++j) acc[i][j] = zero4();

  auto compute = [&](int kt) {
    if (!live) return;
    const int sb = (kt & (C::NST - 1)) * C::STAGE;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const lds_char* A0 = R0 + opaque(aoff[kk] + sb);
      const lds_char* B0 = R0 + opaque(boff[kk] + sb);
      bf16x8_t A[C::FI], Bx[C::TJ];
#pragma unroll
      for (int i = 0; i < C::FI; ++i) A[i] = *(const lds_bf16x8*)(A0 + i * 16 * C::ROWB);
#pragma unroll
      for (int j = 0; j < C::TJ; ++j) Bx[j] = *(const lds_bf16x8*)(B0 + j * 16 * C::ROWB);
#pragma unroll
      for (int i = 0; i < C::FI; ++i)
#pragma unroll
        for (int j = 0; j < C::TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], Bx[j], acc[i][j], 0, 0, 0);
    }
  };

  // Step kt: slices up to kt + NST - 2 are in flight; wait for kt's, then
  // (every wave past the barrier has finished step kt - 1) refill kt - 1's
  // slot with slice kt + NST - 1.
  const int NK = a.D / C::BK;
#pragma unroll
  for (int s = 0; s < C::NST - 1; ++s)
    if (s < NK) issue(s);
  for (int kt = 0; kt < NK; ++kt) {
    wait_slices<C::DPW, C::NST - 2>(NK - 1 - kt);
    barrier();
    if (kt + C::NST - 1 < NK) issue(kt + C::NST - 1);
    compute(kt);
  }

  if (!gen) {
    // q, k, v: four consecutive features of one token per lane, rounded once to bf16
#pragma unroll
    for (int i = 0; i < C::FI; ++i) {
      const int fb = f0 + wf * C::WF + 16 * i;
      if (fb >= 2 * a.Nq + a.Nv) continue;
      bf16_t* out;
      int ld, col;
      if (fb < a.Nq) { out = a.q; ld = a.Nq; col = fb; }
      else if (fb < 2 * a.Nq) { out = a.k; ld = a.Nq; col = fb - a.Nq; }
      else { out = a.v; ld = a.Nv; col = fb - 2 * a.Nq; }
#pragma unroll
      for (int j = 0; j < C::TJ; ++j) {
        const int64_t t = t0 + wt * C::WT + 16 * j + m16;
        if (t >= a.n) continue;
        const f4_t c = acc[i][j];
        uint2 u;
        u.x = (uint32_t)f32_to_bf16(c[0]) | ((uint32_t)f32_to_bf16(c[1]) << 16);
        u.y = (uint32_t)f32_to_bf16(c[2]) | ((uint32_t)f32_to_bf16(c[3]) << 16);
        *reinterpret_cast<uint2*>(out + t * ld + col + 4 * g4) = u;
      }
    }
    return;
  }

  // ---- generator tile: features [W1: 32 | Wa: H (to P) | Wb: H (to P)]
  const int H = a.H, HK = 4 * H;
  barrier();  // every wave is done with the ring
  float (*hid)[GH + 1] = reinterpret_cast<float (*)[GH + 1]>(ring);              // SiLU(W1 x + b1), 64 tokens
  float (*w2s)[GH + 1] = reinterpret_cast<float (*)[GH + 1]>(ring + 64 * (GH + 1) * 4);  // W2 (4H <= 128 rows)
  if (a.taps)
    for (int e = tid; e < HK * GH; e += C::NTHR) w2s[e / GH][e % GH] = bf16_to_f32(a.W2[e]);
  // gates straight from the accumulators
#pragma unroll
  for (int i = 0; i < C::FI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = wf * C::WF + 16 * i + 4 * g4 + r;
      if (f < GH || f >= GH + 2 * P) continue;
      const bool isa = f < GH + P;
      const int h = isa ? f - GH : f - GH - P;
      if (h >= H) continue;
      const bf16_t* bias = isa ? a.ba : a.bb;
      const float bv = bias ? bf16_to_f32(bias[h]) : 0.f;
      float* out = isa ? a.alpha : a.beta;
#pragma unroll
      for (int j = 0; j < C::TJ; ++j) {
        const int64_t t = t0 + wt * C::WT + 16 * j + m16;
        if (t < a.n) out[t * H + h] = 1.0f / (1.0f + expf(-(acc[i][j][r] + bv)));
      }
    }
  // taps, 64 tokens at a time: the hidden layer through LDS, then W2
  constexpr int PT = C::BT < 64 ? C::BT : 64;
  for (int p = 0; p < C::BT && a.taps; p += PT) {
    barrier();  // w2s written; the previous pass's reads of hid done
#pragma unroll
    for (int j = 0; j < C::TJ; ++j) {
      const int tl = wt * C::WT + 16 * j + m16;
      if (tl < p || tl >= p + PT) continue;
#pragma unroll
      for (int i = 0; i < C::FI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = wf * C::WF + 16 * i + 4 * g4 + r;
          if (f >= GH) continue;
          const float hv = acc[i][j][r] + (a.b1 ? bf16_to_f32(a.b1[f]) : 0.f);
          hid[tl - p][f] = hv / (1.0f + expf(-hv));
        }
    }
    barrier();
    for (int e = tid; e < PT * HK; e += C::NTHR) {
      const int tl = e / HK, r = e % HK;
      const int64_t t = t0 + p + tl;
      if (t >= a.n) continue;
      float s = a.b2 ? bf16_to_f32(a.b2[r]) : 0.f;
#pragma unroll 8
      for (int u = 0; u < GH; ++u) s += w2s[r][u] * hid[tl][u];
      a.taps[t * HK + r] = s;
    }
  }
}

// large token counts: 256 x 256 tiles, 8 waves of 128 tokens x 64 features, 64-deep
// slices, two in the ring (measured best of the 256 x 256 shapes at the 2B and 4B widths)
using CfgLarge = Cfg<256, 256, 128, 64, 64, 2, 4, 1>;
// few tokens (decode batches): 64 x 64 tiles, 4 waves of 32 x 32, two workgroups per CU
using CfgSmall = Cfg<64, 64, 32, 32, 64, 4, 4, 2>;

template <class C>
hipError_t run(ProjArgs a, hipStream_t stream) {
  const int nqkv = 2 * a.Nq + a.Nv;
  a.nft = (nqkv + C::BF - 1) / C::BF;
  a.ntf = a.nft + (a.W1 ? 1 : 0);
  a.mtiles = (int)((a.n + C::BT - 1) / C::BT);
  const int64_t total = (int64_t)a.mtiles * a.ntf;
  proj_kernel<C><<<dim3((unsigned)total), dim3(C::NTHR), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

size_t project_workspace_bytes(int64_t, int, int) { return 0; }

hipError_t launch_project(int64_t n, int H, int dk, int dv, int D, const void* x, const void* Wq, const void* Wk,
                          const void* Wv, const void* Wa, const void* ba, const void* Wb, const void* bb,
                          const void* W1, const void* b1, const void* W2, const void* b2, void* q, void* k, void* v,
                          float* alpha, float* beta, float* taps, void*, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (D % 128 || H > 32 || (H * dk) % 32 || (H * dv) % 32) return hipErrorInvalidValue;
  ProjArgs a{};
  a.x = (const bf16_t*)x;
  a.n = n;
  a.D = D; a.H = H; a.Nq = H * dk; a.Nv = H * dv;
  a.Wq = (const bf16_t*)Wq; a.Wk = (const bf16_t*)Wk; a.Wv = (const bf16_t*)Wv;
  a.W1 = (const bf16_t*)W1; a.Wa = (const bf16_t*)Wa; a.Wb = (const bf16_t*)Wb;
  a.b1 = (const bf16_t*)b1; a.W2 = (const bf16_t*)W2; a.b2 = (const bf16_t*)b2;
  a.ba = (const bf16_t*)ba; a.bb = (const bf16_t*)bb;
  a.q = (bf16_t*)q; a.k = (bf16_t*)k; a.v = (bf16_t*)v;
  a.alpha = alpha; a.beta = beta; a.taps = taps;
  return n >= 4096 ? run<CfgLarge>(a, stream) : run<CfgSmall>(a, stream);
}

}  // namespace jb
