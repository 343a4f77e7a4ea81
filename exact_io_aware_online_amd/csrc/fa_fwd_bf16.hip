// fa_fwd_bf16.hip - prefill / training forward in bf16 for gfx950.
//
// One workgroup owns one tile of BM query rows of one (batch, query head)
// and streams every key/value tile it may see (FlashAttention: Part 2,
// section 1.2: query-row tiles are independent units of work; section 1.3:
// each wavefront owns whole rows so no partial results cross wavefronts).
// Per key tile (FlashAttention: Part 2, section 6.2): score tile ->
// online softmax -> value accumulation -> discard; the N x N matrix never
// leaves registers.
//
// The score tile is computed transposed, S^T = K Q^T, with the 32x32x16
// bf16 MFMA: its accumulator puts one query per lane (lane % 32), so each
// lane's running max, running sum and output column belong to a single
// query and the row reductions are in-lane plus one exchange with the lane
// 32 away. The probabilities P^T then feed O^T += V^T P^T directly as the
// B operand, with no trip through LDS. K tiles sit in LDS row-major; V tiles
// are written to LDS transposed (dimension-major) with the key order
// permuted to match where the accumulator left each probability.
//
// Softmax runs in base 2: t = s * scale * log2(e), running maximum m in the
// same units, alpha = 2^(m - m') (FlashAttention: Part 2, section 6.2 gives
// alpha = e^(m - m'); the two agree because e^x = 2^(x log2 e)).
// Normalisation is deferred to the end (FlashAttention: Part 2, section
// 1.3), where the row's log-sum-exp is written as ln2 * (m + log2 l).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

struct FwdParams {
  const bf16* __restrict__ q;
  const bf16* __restrict__ k;
  const bf16* __restrict__ v;
  bf16* __restrict__ o;
  float* __restrict__ lse;
  int Nq, Nk, Hq, Hkv, group;
  int causal;
  int n_qtiles;
  float c;  // scale * log2(e)
};

template <int D, int BN, int NW>
struct Tile {
  static constexpr int BM = NW * 32;          // query rows per workgroup
  static constexpr int THREADS = NW * 64;
  static constexpr int KS = D + 8;            // K row stride in LDS (bf16), padded
  static constexpr int VS = BN + 8;           // V^T row stride in LDS (bf16), padded
  static constexpr int LDS_K = BN * KS;
  static constexpr int LDS_V = D * VS;
  static constexpr int K_CHUNKS = BN * D / 8;             // 16-byte pieces of a K tile
  static constexpr int K_ITERS = (K_CHUNKS + THREADS - 1) / THREADS;
  static constexpr int V_UNITS = (BN / 4) * (D / 8);      // 4 keys x 8 dims each
  static constexpr int V_ITERS = (V_UNITS + THREADS - 1) / THREADS;
  static_assert(BN % 32 == 0, "key tile must be a multiple of 32");
  static_assert(D % 32 == 0, "head dim must be a multiple of 32");
};

// Slot of the first of four consecutive keys (4*kg .. 4*kg+3, kg < 4) of a
// 16-key block inside the transposed V tile. The S^T accumulator leaves key
// 8*(i/4) + 4*g + (i%4) of each 16-key half in register i of lane half g;
// storing that key at slot 8*g + i makes every lane's eight B-operand keys
// contiguous in LDS.
__device__ __forceinline__ int vt_slot(int kg) { return ((kg & 1) << 3) | ((kg >> 1) << 2); }

template <int D, int BN, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdParams p) {
  using T = Tile<D, BN, NW>;
  __shared__ __attribute__((aligned(16))) bf16 smem[T::LDS_K + T::LDS_V];
  bf16* Ks = smem;
  bf16* Vt = smem + T::LDS_K;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;   // which half of the wavefront
  const int r32 = lane & 31; // query within the wavefront's 32 rows

  int qt = blockIdx.x;
  if (p.causal) qt = p.n_qtiles - 1 - qt;  // longest rows first
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = hq / p.group;
  const int q0 = qt * T::BM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + r32;

  const int64_t q_stride = (int64_t)p.Hq * D;   // elements between query rows
  const int64_t kv_stride = (int64_t)p.Hkv * D; // elements between key rows

  // Q^T as the B operand: register i of k-step ks holds Q[my_q][16 ks + 8 g + i].
  bf16x8 qf[D / 16];
  {
    const bf16* qrow = p.q + ((int64_t)b * p.Nq + my_q) * q_stride + (int64_t)hq * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      if (my_q < p.Nq) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + g * 8);
      } else {
        qf[ks] = bf16x8{};
      }
    }
  }

  int kend = p.Nk;
  if (p.causal) kend = min(kend, q0 + T::BM);
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  float m = -INFINITY;  // running max of t, base-2 units
  float l = 0.f;        // running sum of 2^(t - m) over this lane's keys

  const bf16* kbase = p.k + (int64_t)b * p.Nk * kv_stride + (int64_t)kvh * D;
  const bf16* vbase = p.v + (int64_t)b * p.Nk * kv_stride + (int64_t)kvh * D;

  u32x4 kreg[T::K_ITERS];
  u32x4 vreg[T::V_ITERS][4];

  auto load_tile = [&](int j0) {
#pragma unroll
    for (int it = 0; it < T::K_ITERS; ++it) {
      const int c = tid + it * T::THREADS;
      const int row = c / (D / 8), col = c % (D / 8);
      const int key = j0 + row;
      if (c < T::K_CHUNKS && key < p.Nk) {
        kreg[it] = load_u32x4(kbase + (int64_t)key * kv_stride + col * 8);
      } else {
        kreg[it] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int it = 0; it < T::V_ITERS; ++it) {
      const int u = tid + it * T::THREADS;
      const int kg = u % (BN / 4), dc = u / (BN / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j0 + kg * 4 + r;
        if (u < T::V_UNITS && key < p.Nk) {
          vreg[it][r] = load_u32x4(vbase + (int64_t)key * kv_stride + dc * 8);
        } else {
          vreg[it][r] = u32x4{0, 0, 0, 0};
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < T::K_ITERS; ++it) {
      const int c = tid + it * T::THREADS;
      if (c < T::K_CHUNKS) {
        const int row = c / (D / 8), col = c % (D / 8);
        store_u32x4(Ks + row * T::KS + col * 8, kreg[it]);
      }
    }
#pragma unroll
    for (int it = 0; it < T::V_ITERS; ++it) {
      const int u = tid + it * T::THREADS;
      if (u < T::V_UNITS) {
        const int kg = u % (BN / 4), dc = u / (BN / 4);
        const int slot = (kg >> 2) * 16 + vt_slot(kg & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int w = j >> 1;
          uint32_t lo, hi;
          if (j & 1) {
            lo = (vreg[it][0][w] >> 16) | (vreg[it][1][w] & 0xffff0000u);
            hi = (vreg[it][2][w] >> 16) | (vreg[it][3][w] & 0xffff0000u);
          } else {
            lo = (vreg[it][0][w] & 0xffffu) | (vreg[it][1][w] << 16);
            hi = (vreg[it][2][w] & 0xffffu) | (vreg[it][3][w] << 16);
          }
          *reinterpret_cast<u32x2*>(Vt + (dc * 8 + j) * T::VS + slot) = u32x2{lo, hi};
        }
      }
    }
  };

  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * BN;
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();  // the tile is in LDS
    if (t + 1 < ntiles) load_tile(j0 + BN);  // in flight during the math below

    // keys of this tile all lie beyond every query of this wavefront
    if (p.causal && j0 > qw0 + 31) continue;
    const bool need_mask = (j0 + BN > p.Nk) || (p.causal && j0 + BN - 1 > qw0);

    // S^T = K Q^T for BN keys x 32 queries
    f32x16 s[BN / 32];
#pragma unroll
    for (int nb = 0; nb < BN / 32; ++nb) {
      s[nb] = f32x16{};
      const bf16* krow = Ks + (nb * 32 + r32) * T::KS + g * 8;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + ks * 16);
        s[nb] = mfma32x32x16(kf, qf[ks], s[nb]);
      }
    }

    if (need_mask) {
#pragma unroll
      for (int nb = 0; nb < BN / 32; ++nb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + nb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= p.Nk || (p.causal && key > my_q)) s[nb][i] = -INFINITY;
        }
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < BN / 32; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[nb][i]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m, mx * p.c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // no (-inf) - (-inf)
    const float alpha = exp2_fast(m - m_use);
    m = m_new;

    float rs = 0.f;
#pragma unroll
    for (int nb = 0; nb < BN / 32; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = exp2_fast(fmaf(s[nb][i], p.c, -m_use));
        s[nb][i] = pv;
        rs += pv;
      }
    l = fmaf(l, alpha, rs);

    // P^T as B operands: 16-key step kk takes registers 8*(kk%2) .. +7 of
    // accumulator kk/2 (keys 8*(i/4) + 4g + i%4 of that 16-key half).
    bf16x8 pf[BN / 16];
#pragma unroll
    for (int kk = 0; kk < BN / 16; ++kk) {
      const int nb = kk >> 1, h = (kk & 1) * 8;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(s[nb][h + 2 * e], s[nb][h + 2 * e + 1]);
      pf[kk] = __builtin_bit_cast(bf16x8, w);
    }

#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const bf16* vrow = Vt + (dt * 32 + r32) * T::VS + g * 8;
#pragma unroll
      for (int kk = 0; kk < BN / 16; ++kk) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vrow + kk * 16);
        acc[dt] = mfma32x32x16(vf, pf[kk], acc[dt]);
      }
    }
  }

  // Epilogue: combine the two lane halves' partial sums, normalise once.
  const float lt = l + swap_halves(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (my_q < p.Nq) {
    bf16* orow = p.o + ((int64_t)b * p.Nq + my_q) * q_stride + (int64_t)hq * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = dt * 32 + 8 * j + 4 * g;
        u32x2 w;
        w[0] = pack_bf16x2(acc[dt][4 * j + 0] * inv, acc[dt][4 * j + 1] * inv);
        w[1] = pack_bf16x2(acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    }
    if (p.lse != nullptr && g == 0) {
      p.lse[((int64_t)b * p.Hq + hq) * p.Nq + my_q] = lt > 0.f ? (m + log2_fast(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int BN, int NW>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  using T = Tile<D, BN, NW>;
  FwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.o = static_cast<bf16*>(a.o);
  p.lse = a.lse;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.causal = a.causal;
  p.n_qtiles = (a.Nq + T::BM - 1) / T::BM;
  p.c = a.scale * kLog2e;
  dim3 grid(p.n_qtiles, a.Hq, a.B);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, NW>), grid, dim3(T::THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool fwd_bf16_supported(int d) { return d == 64 || d == 128 || d == 256; }

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch<64, 64, 4>(a, stream);
    case 128: return launch<128, 64, 4>(a, stream);
    case 256: return launch<256, 32, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
