// fa_fp8.hip - FP8 (e4m3) forward for gfx950: block quantisation with an
// optional randomised Hadamard rotation, and attention whose two products
// run on the FP8 MFMA.
//
// FlashAttention: Part 2, section 1.6 "FA3 FP8": converting every operand
// to FP8 with one global scale loses too much; the FP8 path scales each
// tile by its own range (block quantisation) and multiplies Q and K by a
// random orthogonal matrix first (incoherent processing), which spreads
// outlier features over the head dimension; the algorithm is still exact
// softmax(Q K^T) V, only its arithmetic is FP8.
//
// Quantisation (quant_kernel): one workgroup per 64-row block of one
// (batch, head). Optional rotation R = H_d diag(s) / sqrt(d) (H_d the
// Sylvester Hadamard matrix) by a fast Walsh-Hadamard transform over each
// row; then the block's scale 2^e, e the smallest integer with
// amax <= 448 * 2^e, and round-to-nearest-even e4m3 codes of x * 2^-e.
// Power-of-two scales make the scaling exact and feed the MFMA's E8M0
// scale operands directly. Codes are written per head in the layout the
// attention kernel streams: (B, H, Np, d) for Q and K, (B, H, d, Np) for V
// (transposed, so each lane's 32 keys of a V^T operand are contiguous).
//
// Attention (fwd_fp8_kernel): the bf16 kernel's structure (one workgroup
// per 128 query rows, 64-key K and V^T tiles in a direct-to-LDS ring, one
// query per lane of S^T = K Q^T) on v_mfma_scale_f32_32x32x64_f8f6f4:
// S^T with the K tile's and the Q block's E8M0 scales, O^T += V^T P^T with
// the V tile's scale. The 32 keys a lane holds in S^T become exactly the
// 32 bytes of its P^T operand because the K operand rows are read in a
// permuted order (row m of 32-key block b is key
// 32 ((m / 4) % 2) + 16 b + 4 (m / 8) + m % 4 of the tile), so lane half h
// holds keys 32 h .. 32 h + 31 and reads the same 32 contiguous keys of
// V^T. The probabilities are quantised as e4m3 of 2^(t - m + 6) against an
// integer running maximum m (base-2 units, moved only when the row maximum
// grew by more than 2): rescaling is then by exact powers of two and each
// probability's code does not depend on when m moved. The denominator sums
// the unquantised probabilities.
#include <stdlib.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kRows = kFp8Block;  // rows per quantisation block and per key tile
constexpr int kPBias = 6;         // probabilities are quantised as e4m3(2^(t - m + kPBias))
constexpr float kSlack2 = 2.f;    // growth of a row maximum tolerated before m moves

__device__ __forceinline__ uint32_t cvt_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// ---------------------------------------------------------------------------
// quantisation
// ---------------------------------------------------------------------------
struct QuantParams {
  const char* __restrict__ x;       // (B, N, H, D) bf16
  const float* __restrict__ signs;  // (D,) +-1, or null: no rotation
  uint8_t* __restrict__ codes;      // (B, H, Np, D), or (B, H, D, Np) transposed
  uint8_t* __restrict__ scales;     // (B, H, Np / 64) E8M0 (127 + e)
  int N, Np, H;
};

template <int D, bool TRANS>
__global__ __launch_bounds__(256) void quant_kernel(QuantParams p) {
  constexpr int E = D / 4;  // elements per thread: a quarter of a row
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[TRANS ? kRows * D : 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = tid >> 2, part = tid & 3;
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = blk * kRows + r;

  float x[E];
  if (n < p.N) {
    const char* src = p.x + (((int64_t)b * p.N + n) * p.H + h) * D * 2 + part * E * 2;
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + i * 16);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[8 * i + j] = (float)v[j];
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = 0.f;
  }

  if (p.signs != nullptr) {
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] *= p.signs[part * E + i];
    // Walsh-Hadamard butterflies (a, c) -> (a + c, a - c): strides below E
    // inside the thread, strides E and 2E across the row's four threads
#pragma unroll
    for (int s = 1; s < E; s <<= 1)
#pragma unroll
      for (int i = 0; i < E; ++i)
        if ((i & s) == 0) {
          const float a = x[i], c = x[i + s];
          x[i] = a + c;
          x[i + s] = a - c;
        }
#pragma unroll
    for (int s = 1; s <= 2; s <<= 1) {
      const bool upper = (part & s) != 0;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float o = __shfl_xor(x[i], s, 64);
        x[i] = upper ? o - x[i] : x[i] + o;
      }
    }
    const float inv = 1.f / __builtin_sqrtf((float)D);
    // padding rows stay +0 (the butterflies of zeros can leave -0)
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = n < p.N ? x[i] * inv : 0.f;
  }

  // block maximum |x| and its power-of-two scale
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) am = fmaxf(am, fabsf(x[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
  if (lane == 0) red[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (am > 0.f) {
    int ex;
    const float f = frexpf(am, &ex);  // am = f 2^ex, f in [0.5, 1); 448 = 0.875 2^9
    e = f <= 0.875f ? ex - 9 : ex - 8;
    e = min(max(e, -127), 127);
  }

  uint32_t w[E / 4];
#pragma unroll
  for (int i = 0; i < E / 4; ++i)
    w[i] = cvt_fp8x4(ldexpf(x[4 * i], -e), ldexpf(x[4 * i + 1], -e), ldexpf(x[4 * i + 2], -e),
                     ldexpf(x[4 * i + 3], -e));

  const int64_t head = (int64_t)b * p.H + h;
  if (tid == 0) p.scales[head * (p.Np / kRows) + blk] = (uint8_t)(e + 127);
  if constexpr (!TRANS) {
    uint8_t* dst = p.codes + (head * p.Np + n) * D + part * E;
#pragma unroll
    for (int i = 0; i < E / 16; ++i)
      *reinterpret_cast<u32x4*>(dst + 16 * i) = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  } else {
    // through LDS: row-major block in, one dimension's run of rows out
#pragma unroll
    for (int i = 0; i < E / 4; ++i) *reinterpret_cast<uint32_t*>(tile + r * D + part * E + 4 * i) = w[i];
    __syncthreads();
    constexpr int TPD = 256 / D;     // threads per dimension
    constexpr int RPT = kRows / TPD;  // rows per thread
    const int dim = tid / TPD, r0 = (tid % TPD) * RPT;
    uint32_t o[RPT / 4];
#pragma unroll
    for (int i = 0; i < RPT / 4; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) v |= (uint32_t)tile[(r0 + 4 * i + k) * D + dim] << (8 * k);
      o[i] = v;
    }
    uint8_t* dst = p.codes + (head * D + dim) * p.Np + blk * kRows + r0;
#pragma unroll
    for (int i = 0; i < RPT / 16; ++i)
      *reinterpret_cast<u32x4*>(dst + 16 * i) = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
  }
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
struct Fp8Params {
  const uint8_t* __restrict__ q;   // (B, Hq, Nqp, D) codes
  const uint8_t* __restrict__ k;   // (B, Hkv, Nkp, D)
  const uint8_t* __restrict__ vt;  // (B, Hkv, D, Nkp)
  const uint8_t* __restrict__ qs;  // (B, Hq, Nqp / 64) E8M0
  const uint8_t* __restrict__ ks;  // (B, Hkv, Nkp / 64)
  const uint8_t* __restrict__ vs;
  char* __restrict__ o;            // (B, Nq, Hq, D) bf16
  float* __restrict__ lse;         // (B, Hq, Nq) or null
  int Nq, Nk, Nqp, Nkp, Hq, Hkv, group, B, causal, n_qtiles;
  float c;  // scale * log2(e)
};

template <int D_, int NST_, int WPS_>
struct F8Cfg {
  static constexpr int D = D_, NST = NST_, WPS = WPS_;
  static constexpr int BN = 64, NW = 4, BM = NW * 32, THREADS = NW * 64;
  static constexpr int TILE = BN * D;            // bytes of a K tile and of a V^T tile
  static constexpr int V_REGION = NST * TILE;    // K tiles, then V^T tiles
  static constexpr int DMA = TILE / (THREADS * 16);
  static_assert(D == 64 || D == 128 || D == 256, "head dimension");
  static_assert(DMA >= 1 && TILE % (THREADS * 16) == 0, "tile does not split over the threads");
  static_assert(NST >= 2 && (NST - 2) * 2 * DMA <= 63, "vmcnt range");
  // the S = K Q^T block also runs at raised issue priority: at d = 256 its 16
  // K operand reads per MFMA chain otherwise queue behind the other wave's
  // exponentials (about 2% on a long non-causal d = 256 prefill; neutral to
  // slightly slower at d = 64 and 128)
  static constexpr bool PRIO_S = D == 256;
  // ring stage as an immediate LDS offset (one copy of the tile code per
  // stage); at d = 256 the copies' register allocation keeps two versions
  // of the accumulators, so there the stage is a register
  static constexpr bool CONST_STAGE = D < 256;
};

// 16-byte chunk swizzle of a K tile row (D bytes = D / 16 chunks): the 16
// rows one quarter-wave reads together (keys {0..3, 32..35, 4..7, 36..39}
// of a 32-key block, plus 8) land in distinct 16-byte bank groups of the
// 256-byte bank window (2 rows of 128 bytes, 4 of 64, 1 of 256)
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 64) return ((row >> 2) & 1) | (((row >> 5) & 1) << 1);
  else if constexpr (D == 128) return ((row >> 1) & 3) | (((row >> 5) & 1) << 2);
  else return (row & 7) | (((row >> 5) & 1) << 3);
}
// and of a V^T tile row (64 bytes = 4 chunks)
__device__ __forceinline__ int swz_v(int dim) { return (dim >> 2) & 3; }

__device__ __forceinline__ i32x8 lds_read32(uint32_t a0, uint32_t a1) {
  const u32x4 x = *(const LDS3 u32x4*)(uintptr_t)a0;
  const u32x4 y = *(const LDS3 u32x4*)(uintptr_t)a1;
  return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

template <class C>
__global__ __launch_bounds__(C::THREADS, C::WPS) void fwd_fp8_kernel(Fp8Params p) {
  constexpr int D = C::D, NST = C::NST, BN = C::BN;
  __shared__ __attribute__((aligned(1024))) char smem[2 * NST * C::TILE];
  __shared__ uint8_t sc_k[kFp8MaxKeys / kRows], sc_v[kFp8MaxKeys / kRows];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS3 char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int r32 = lane & 31;

  // work order as in the bf16 kernel: query-tile rank outermost (longest
  // causal tiles first), the query heads of one key/value head a multiple
  // of Hkv * B apart (same XCD)
  const int heads = p.Hq * p.B;
  const int rk = blockIdx.x / heads;
  const int rest = blockIdx.x - rk * heads;
  const int pairs = p.Hkv * p.B;
  const int jg = rest / pairs;
  const int pr = rest - jg * pairs;
  const int b = pr / p.Hkv;
  const int kvh = pr - b * p.Hkv;
  const int hq = kvh * p.group + jg;
  const int qt = p.causal ? p.n_qtiles - 1 - rk : rk;
  const int q0 = qt * C::BM;
  const int qw0 = q0 + wave * 32;
  const int q_last = min(q0 + C::BM, p.Nq) - 1;
  const int khi = p.causal ? min(q_last, p.Nk - 1) : p.Nk - 1;
  const int ntiles = khi >= 0 ? khi / BN + 1 : 0;

  const int64_t kvhead = (int64_t)b * p.Hkv + kvh;
  const uint8_t* kbase = p.k + kvhead * p.Nkp * D;
  const uint8_t* vbase = p.vt + kvhead * D * p.Nkp;
  uint32_t k_dma[C::DMA], v_dma[C::DMA];
#pragma unroll
  for (int j = 0; j < C::DMA; ++j) {
    const int slot = j * C::THREADS + tid;
    const int row = slot / (D / 16), kc = (slot % (D / 16)) ^ swz_k<D>(row);
    k_dma[j] = (uint32_t)(row * D + 16 * kc);
    const int dim = slot / 4, vc = (slot % 4) ^ swz_v(dim);
    v_dma[j] = (uint32_t)(dim * p.Nkp + 16 * vc);
  }
  const uint32_t dma_lds = __builtin_amdgcn_readfirstlane(lds0 + wave * 64 * 16);
  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    const uint8_t* ks = kbase + (int64_t)t * BN * D;
    const uint8_t* vs = vbase + t * BN;
    const uint32_t st = dma_lds + (uint32_t)((t % NST) * C::TILE);
#pragma unroll
    for (int j = 0; j < C::DMA; ++j) dma16(ks, k_dma[j], st + j * C::THREADS * 16);
#pragma unroll
    for (int j = 0; j < C::DMA; ++j) dma16(vs, v_dma[j], st + C::V_REGION + j * C::THREADS * 16);
  };
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < ntiles) issue_tile(s);

  // the tiles' E8M0 scales into LDS; the wavefront's Q block scale and its
  // Q^T operands (lane half g supplies dimensions 64 s + 32 g .. + 31)
  for (int i = tid; i < ntiles; i += C::THREADS) {
    sc_k[i] = p.ks[kvhead * (p.Nkp / kRows) + i];
    sc_v[i] = p.vs[kvhead * (p.Nkp / kRows) + i];
  }
  const int64_t qhead = (int64_t)b * p.Hq + hq;
  const int qsc = qw0 < p.Nqp ? (int)p.qs[qhead * (p.Nqp / kRows) + qw0 / kRows] : 127;
  i32x8 qf[D / 64];
  {
    const int row = qw0 + r32;
    const uint8_t* qrow = p.q + (qhead * p.Nqp + row) * D + 32 * g;
#pragma unroll
    for (int s = 0; s < D / 64; ++s) {
      if (row < p.Nqp) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 64 * s);
        const u32x4 y = *reinterpret_cast<const u32x4*>(qrow + 64 * s + 16);
        qf[s] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
      } else {
        qf[s] = i32x8{};
      }
    }
  }
  wait_vm_loads();
  __syncthreads();  // the scale bytes are visible to every wavefront

  // LDS read offsets: K operand rows in the permuted key order, V^T rows.
  // Neither swizzle looks at the row bits that the 16-key block nb (bit 4
  // of the K row) or the 32-dimension block dt (bits 5 and up of the V^T
  // row) set, so those blocks are a constant apart: registers for nb = 0
  // and dt = 0, the rest immediates.
  uint32_t k_off[D / 64][2];
  {
    const int kr = 32 * ((r32 >> 2) & 1) + 4 * (r32 >> 3) + (r32 & 3);
#pragma unroll
    for (int s = 0; s < D / 64; ++s)
#pragma unroll
      for (int e = 0; e < 2; ++e) k_off[s][e] = (uint32_t)(kr * D + 16 * ((4 * s + 2 * g + e) ^ swz_k<D>(kr)));
  }
  auto kofs = [&](int nb, int s, int e) __attribute__((always_inline)) { return k_off[s][e] + (uint32_t)(nb * 16 * D); };
  uint32_t v_off[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) v_off[e] = (uint32_t)(C::V_REGION + r32 * BN + 16 * ((2 * g + e) ^ swz_v(r32)));
  auto vofs = [&](int dt, int e) __attribute__((always_inline)) { return v_off[e] + (uint32_t)(dt * 32 * BN); };

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  float m = -INFINITY;  // running maximum of t, an integer (base-2 units)
  float l = 0.f;        // running sum of 2^(t - m) over this lane's keys

  auto sync_tile = [&](int t) __attribute__((always_inline)) {
    const int after = min(NST - 2, ntiles - 1 - t);
    static_for<NST - 1>([&](auto A) {
      if (after == decltype(A)::value) wait_vmcnt<decltype(A)::value * 2 * C::DMA>();
    });
    barrier();
    if (t + NST - 1 < ntiles) issue_tile(t + NST - 1);
  };

  f32x16 sc[2];
  i32x8 pf;

  auto s_phase = [&](int t, auto stage) __attribute__((always_inline)) {
    const uint32_t stg = lds0 + (uint32_t)(int)stage * C::TILE;
    const int ksc = sc_k[t];
    sc[0] = f32x16{};
    sc[1] = f32x16{};
    if constexpr (D <= 128) {  // every K operand read ahead of the chain
      i32x8 kf[2][D / 64];
#pragma unroll
      for (int s = 0; s < D / 64; ++s)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) kf[nb][s] = lds_read32(stg + kofs(nb, s, 0), stg + kofs(nb, s, 1));
#pragma unroll
      for (int s = 0; s < D / 64; ++s)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) sc[nb] = mfma_fp8(kf[nb][s], qf[s], sc[nb], ksc, qsc);
    } else {  // d = 256: one slab's operands at a time (registers)
#pragma unroll
      for (int s = 0; s < D / 64; ++s) {
        i32x8 kf[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) kf[nb] = lds_read32(stg + kofs(nb, s, 0), stg + kofs(nb, s, 1));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) sc[nb] = mfma_fp8(kf[nb], qf[s], sc[nb], ksc, qsc);
      }
    }
  };

  auto softmax_phase = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (MASK) {
      // register i of block nb holds key t BN + 32 g + 16 nb + i
      const int my_q = qw0 + r32;
      const int lim = (p.causal ? min(my_q, p.Nk - 1) : p.Nk - 1) - t * BN - 32 * g;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * nb + i > lim) sc[nb][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[nb][i]);
    mx = halves_max(mx);
    const float m_cand = fmaxf(m, mx * p.c);
    const bool rescale = __builtin_amdgcn_ballot_w64(m_cand > m + kSlack2) != 0;
    float alpha = 1.f;
    if (rescale) {
      const float m_new = m_cand == -INFINITY ? -INFINITY : ceilf(m_cand);
      alpha = m == -INFINITY ? 0.f : ldexpf(1.f, (int)(m - m_new));  // exact power of two
      l *= alpha;
      m = m_new;
    }
    const float mb = (m == -INFINITY) ? 0.f : m - (float)kPBias;
    float e[32];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = exp2_fast(fmaf(sc[nb][i], p.c, -mb));
        sc[nb][i] = pv;
        e[16 * nb + i] = pv;
      }
#pragma unroll
    for (int w = 16; w >= 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) e[i] += e[i + w];
    l += e[0] * (1.f / (1 << kPBias));
    // P^T operand: byte j of lane half g is key 32 g + j = register j % 16 of block j / 16
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int nb = w >> 2, i0 = 4 * (w & 3);
      pf[w] = (int)cvt_fp8x4(sc[nb][i0], sc[nb][i0 + 1], sc[nb][i0 + 2], sc[nb][i0 + 3]);
    }
    if (rescale) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
    }
  };

  auto pv_phase = [&](int t, auto stage) __attribute__((always_inline)) {
    const uint32_t stg = lds0 + (uint32_t)(int)stage * C::TILE;
    const int vsc = sc_v[t];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const i32x8 vf = lds_read32(stg + vofs(dt, 0), stg + vofs(dt, 1));
      acc[dt] = mfma_fp8(vf, pf, acc[dt], vsc, 127);
      // d = 256: keep each V operand next to its MFMA (registers)
      if constexpr (D > 128) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The compiler puts one wait state fewer between a scaled FP8 MFMA and a
  // 64-bit register move (v_mov_b64) that reads its result than it puts
  // before other vector reads (19 against 20 after
  // v_mfma_scale_f32_32x32x64_f8f6f4). On MI355X such a move, in the
  // accumulator copies the compiler makes where one loop hands over to the
  // next, then read the last two rows of a block before the MFMA had
  // written them (wrong and run-to-run different outputs). Two wait states
  // after each MFMA phase, in inline assembly, which the compiler counts as
  // none, put every later read of the results past its own bound.
  auto mfma_guard = [] __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 1");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute_tile = [&](int t, auto mask_tag, auto stage) __attribute__((always_inline)) {
    if constexpr (C::PRIO_S) {
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
      s_phase(t, stage);
      mfma_guard();
      __builtin_amdgcn_s_setprio(0);
    } else {
      __builtin_amdgcn_sched_barrier(0);
      s_phase(t, stage);
      mfma_guard();
    }
    softmax_phase(t, mask_tag);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    pv_phase(t, stage);
    mfma_guard();
    __builtin_amdgcn_s_setprio(0);
  };
  auto compute_any = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    const int st = t % NST;
    if constexpr (C::CONST_STAGE) {
      static_for<NST>([&](auto S) {
        if (st == decltype(S)::value) compute_tile(t, mask_tag, S);
      });
    } else {
      compute_tile(t, mask_tag, st);
    }
  };

  // this wavefront's tiles: [0, u_hi) unmasked, [u_hi, t_hi) masked, the
  // rest only kept in step with the workgroup's pipeline
  int t_hi = 0, u_hi = 0;
  if (qw0 < p.Nq && p.Nk > 0) {
    const int wq_last = min(qw0 + 31, p.Nq - 1);
    const int whi = p.causal ? min(wq_last, p.Nk - 1) : p.Nk - 1;
    t_hi = min(whi / BN + 1, ntiles);
    const int fhi = p.causal ? min(qw0, p.Nk - 1) : p.Nk - 1;  // every row sees keys <= fhi
    u_hi = min((fhi + 1) / BN, t_hi);
  }
  int t = 0;
  if constexpr (C::CONST_STAGE) {
    for (; t + NST <= u_hi; t += NST) {
      static_for<NST>([&](auto S) {
        sync_tile(t + decltype(S)::value);
        compute_tile(t + decltype(S)::value, std::false_type{}, S);
      });
    }
  }
  for (; t < u_hi; ++t) {
    sync_tile(t);
    compute_any(t, std::false_type{});
  }
  for (; t < t_hi; ++t) {
    sync_tile(t);
    compute_any(t, std::true_type{});
  }
  for (; t < ntiles; ++t) sync_tile(t);

  // epilogue: O = 2^-kPBias acc / l, LSE = ln2 (m + log2 l). As in the bf16
  // kernel, at d = 64 and 128 the rows go through the idle LDS ring so that
  // 16-byte lanes store whole rows (non-temporal: written once, not read
  // here); d = 256 stores from the accumulators.
  constexpr int ROWB = D * 2, CPR = D / 8;
  constexpr bool STAGE_O = D <= 128 && C::NW * 32 * ROWB <= 2 * NST * C::TILE;
  const int my_q = qw0 + r32;
  const float lt = halves_sum(l);
  const float inv = lt > 0.f ? (1.f / (1 << kPBias)) / lt : 0.f;
  if constexpr (STAGE_O) {
    const uint32_t ost = lds0 + (uint32_t)(wave * 32 * ROWB);
    barrier();  // every wavefront is done reading the ring
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = dt * 4 + j;  // 16-byte chunk of dims 8c .. 8c+7; half g holds 8c + 4g ..
        u32x2 w;
        w[0] = pack_bf16x2(acc[dt][4 * j + 0] * inv, acc[dt][4 * j + 1] * inv);
        w[1] = pack_bf16x2(acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv);
        *(LDS3 u32x2*)(uintptr_t)(ost + r32 * ROWB + ((c ^ (r32 % CPR)) * 16) + g * 8) = w;
      }
    if (my_q < p.Nq && p.lse != nullptr && g == 0)
      p.lse[qhead * p.Nq + my_q] = lt > 0.f ? (m + log2_fast(lt)) * kLn2 : -INFINITY;
    // a wavefront reads back only its own rows (its LDS instructions complete in order)
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int slot = i * 64 + lane;
      const int row = slot / CPR, c = slot % CPR;
      const u32x4 w = *(const LDS3 u32x4*)(uintptr_t)(ost + row * ROWB + ((c ^ (row % CPR)) * 16));
      const int q = qw0 + row;
      if (q < p.Nq)
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p.o + (((int64_t)b * p.Nq + q) * p.Hq + hq) * D * 2 +
                                                                c * 16));
    }
  } else {
    // stores straight from the accumulators, in the code shape the d = 256
    // kernel's register allocation was measured with
    if (my_q < p.Nq) {
      char* orow = p.o + (((int64_t)b * p.Nq + my_q) * p.Hq + hq) * D * 2;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d0 = dt * 32 + 8 * j + 4 * g;
          u32x2 w;
          w[0] = pack_bf16x2(acc[dt][4 * j + 0] * inv, acc[dt][4 * j + 1] * inv);
          w[1] = pack_bf16x2(acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d0 * 2) = w;
        }
      if (p.lse != nullptr && g == 0)
        p.lse[qhead * p.Nq + my_q] = lt > 0.f ? (m + log2_fast(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool TRANS>
hipError_t launch_quant(const Fp8QuantArgs& a, hipStream_t stream) {
  QuantParams p;
  p.x = static_cast<const char*>(a.x);
  p.signs = a.signs;
  p.codes = static_cast<uint8_t*>(a.codes);
  p.scales = a.scales;
  p.N = a.N;
  p.Np = fp8_padded_rows(a.N);
  p.H = a.H;
  dim3 grid(p.Np / kRows, a.H, a.B);
  hipLaunchKernelGGL((quant_kernel<D, TRANS>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <class C>
hipError_t launch_fp8(const Fp8FwdArgs& a, hipStream_t stream) {
  Fp8Params p;
  p.q = static_cast<const uint8_t*>(a.q8);
  p.k = static_cast<const uint8_t*>(a.k8);
  p.vt = static_cast<const uint8_t*>(a.vt8);
  p.qs = a.q_scales;
  p.ks = a.k_scales;
  p.vs = a.v_scales;
  p.o = static_cast<char*>(a.o);
  p.lse = a.lse;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.Nqp = fp8_padded_rows(a.Nq);
  p.Nkp = fp8_padded_rows(a.Nk);
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.B = a.B;
  p.causal = a.causal;
  p.n_qtiles = (a.Nq + C::BM - 1) / C::BM;
  p.c = a.scale * kLog2e;
  dim3 grid(p.n_qtiles * a.Hq * a.B);
  hipLaunchKernelGGL((fwd_fp8_kernel<C>), grid, dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int fp8_padded_rows(int n) { return (n + kRows - 1) / kRows * kRows; }
bool fp8_quant_supported(int d) { return d == 64 || d == 128 || d == 256; }
bool fp8_fwd_supported(int d) { return d == 64 || d == 128 || d == 256; }

hipError_t launch_quant_fp8(const Fp8QuantArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return a.transpose ? launch_quant<64, true>(a, stream) : launch_quant<64, false>(a, stream);
    case 128: return a.transpose ? launch_quant<128, true>(a, stream) : launch_quant<128, false>(a, stream);
    case 256: return a.transpose ? launch_quant<256, true>(a, stream) : launch_quant<256, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_fp8<F8Cfg<64, 2, 3>>(a, stream);
    case 128: return launch_fp8<F8Cfg<128, 2, 2>>(a, stream);
    // two wavefronts per SIMD at every head dimension (d = 256 fits 256
    // registers once its ring stage is a register and its LDS offsets are
    // shared: twice as fast as one wavefront per SIMD on MI355X)
    case 256: return launch_fp8<F8Cfg<256, 2, 2>>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
