// fa_decode.hip - split-KV decode and log-sum-exp combine for gfx950.
//
// Decode has one query per sequence, so it streams the key/value cache and
// is bound by memory bandwidth (FlashAttention: Part 2, section 4.1). The
// cache of each sequence is cut into splits that separate workgroups load
// in parallel, and a second kernel merges their partial results
// (pyshine.com FlashAttention code tour, "Why You Need This").
//
// Split kernel: workgroup (split s, key/value head h, sequence b) serves all
// G = Hq / Hkv query heads that read head h, so each cache byte is read
// once. Its 64-key tiles are staged through LDS (K row-major, V transposed)
// by all four wavefronts; wavefront w takes keys 16w .. 16w+15 of each tile
// and keeps its own online-softmax state (FlashAttention: Part 2, section
// 6.2). Scores use S^T = K Q^T on the 16x16x32 bf16 MFMA with the G query
// heads as columns (the other 16 - G columns are zero); the accumulator
// layout is exactly the B-operand layout of the 16x16x16 MFMA, so P^T feeds
// O^T += V^T P^T straight from registers. At the end the four wavefronts'
// states merge through LDS.
//
// Partial results: O_s (normalised, fp32) and L_s = log2 of the split's sum
// of 2^(t) in base-2 units; an empty split is never written, the combine
// derives from the sequence length which splits exist.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kTile = 64;      // keys per LDS tile
constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kMaxGroup = 16;  // query heads per key/value head (MFMA columns)

struct DecParams {
  const bf16* __restrict__ q;
  const bf16* __restrict__ kc;
  const bf16* __restrict__ vc;
  const int32_t* __restrict__ lens;
  bf16* __restrict__ o;
  float* __restrict__ lse;
  float* __restrict__ part_o;    // (B, Hq, S, D)
  float* __restrict__ part_lse;  // (B, Hq, S), base-2 units
  int Hq, Hkv, group, capacity, S, chunk;
  float c;  // scale * log2(e)
};

__device__ __forceinline__ int seq_len(const DecParams& p, int b) {
  return min(max(p.lens[b], 0), p.capacity);
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecParams p) {
  constexpr int KS = D + 8;       // K row stride in LDS (bf16)
  constexpr int VS = kTile + 8;   // V^T row stride in LDS (bf16)
  constexpr int K_ITERS = kTile * D / 8 / kThreads;
  constexpr int V_UNITS = (kTile / 4) * (D / 8);
  constexpr int V_ITERS = (V_UNITS + kThreads - 1) / kThreads;
  static_assert(K_ITERS >= 1 && (kTile * D / 8) % kThreads == 0, "tile/threads mismatch");
  __shared__ __attribute__((aligned(16))) bf16 smem[kTile * KS + D * VS];
  bf16* Ks = smem;
  bf16* Vt = smem + kTile * KS;
  __shared__ float red_m[4][kMaxGroup];
  __shared__ float red_l[4][kMaxGroup];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15;  // query head within the group (MFMA column)
  const int g4 = lane >> 4;   // lane quarter
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = seq_len(p, b);
  const int start = s * p.chunk;
  const int end = min(start + p.chunk, L);
  if (start >= end && !(p.S == 1 && start == 0)) return;  // empty split: nothing to write

  const int G = p.group;
  const int hq = h * G + col;
  const int64_t kv_stride = (int64_t)p.Hkv * D;

  // Q^T as B operand of 16x16x32: register i of k-step ks = Q[hq][32 ks + 8 g4 + i].
  bf16x8 qf[D / 32];
  {
    const bf16* qrow = p.q + ((int64_t)b * p.Hq + hq) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[ks] = col < G ? *reinterpret_cast<const bf16x8*>(qrow + ks * 32 + g4 * 8) : bf16x8{};
  }

  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{};
  float m = -INFINITY, l = 0.f;

  const bf16* kbase = p.kc + (int64_t)b * p.capacity * kv_stride + (int64_t)h * D;
  const bf16* vbase = p.vc + (int64_t)b * p.capacity * kv_stride + (int64_t)h * D;
  u32x4 kreg[K_ITERS];
  u32x4 vreg[V_ITERS][4];

  auto load_tile = [&](int j0) {
#pragma unroll
    for (int it = 0; it < K_ITERS; ++it) {
      const int c = tid + it * kThreads;
      const int row = c / (D / 8), cc = c % (D / 8);
      const int key = j0 + row;
      kreg[it] = key < end ? load_u32x4(kbase + (int64_t)key * kv_stride + cc * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < V_ITERS; ++it) {
      const int u = tid + it * kThreads;
      const int kg = u % (kTile / 4), dc = u / (kTile / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j0 + kg * 4 + r;
        vreg[it][r] = (u < V_UNITS && key < end) ? load_u32x4(vbase + (int64_t)key * kv_stride + dc * 8)
                                                 : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < K_ITERS; ++it) {
      const int c = tid + it * kThreads;
      store_u32x4(Ks + (c / (D / 8)) * KS + (c % (D / 8)) * 8, kreg[it]);
    }
#pragma unroll
    for (int it = 0; it < V_ITERS; ++it) {
      const int u = tid + it * kThreads;
      if (u < V_UNITS) {
        const int kg = u % (kTile / 4), dc = u / (kTile / 4);
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
          *reinterpret_cast<u32x2*>(Vt + (dc * 8 + j) * VS + kg * 4) = u32x2{lo, hi};
        }
      }
    }
  };

  const int ntiles = (end - start + kTile - 1) / kTile;
  if (ntiles > 0) load_tile(start);
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = start + t * kTile;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(j0 + kTile);

    const int kw0 = j0 + wave * 16;  // first key of this wavefront
    if (kw0 >= end) continue;

    // S^T (16 keys x 16 columns)
    f32x4 sc = f32x4{};
    const bf16* krow = Ks + (wave * 16 + col) * KS + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + ks * 32);
      sc = mfma16x16x32(kf, qf[ks], sc);
    }
    // lane (col, g4) holds keys kw0 + 4 g4 + i
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (kw0 + 4 * g4 + i >= end) sc[i] = -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx * p.c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_use);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = exp2_fast(fmaf(sc[i], p.c, -m_use));
      rs += sc[i];
    }
    l = fmaf(l, alpha, rs);
    i16x4 pf;
    {
      const uint32_t w0 = pack_bf16x2(sc[0], sc[1]), w1 = pack_bf16x2(sc[2], sc[3]);
      pf = __builtin_bit_cast(i16x4, u32x2{w0, w1});
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      acc[dt] *= alpha;
      const i16x4 vf = *reinterpret_cast<const i16x4*>(Vt + (dt * 16 + col) * VS + wave * 16 + g4 * 4);
      acc[dt] = mfma16x16x16(vf, pf, acc[dt]);
    }
  }

  // Merge the four wavefronts: sum l over lane quarters, then across waves.
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (g4 == 0 && col < kMaxGroup) {
    red_m[wave][col] = m;
    red_l[wave][col] = l;
  }
  __syncthreads();  // also: every wave is done with the K/V tiles
  float* red_o = reinterpret_cast<float*>(smem);  // reuse the tile memory: 4 x 16 x D floats
  static_assert(4 * kMaxGroup * D * 4 <= (kTile * KS + D * VS) * 2, "merge buffer too small");
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][col]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  const float my_w = exp2_fast(m - Mu);
  // lane (col, g4) holds O^T[d = 16 dt + 4 g4 + i][col]
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_o[(wave * kMaxGroup + col) * D + dt * 16 + 4 * g4 + i] = acc[dt][i] * my_w;
  __syncthreads();

  // Thread layout for the output: query column qc, dimensions d..d+dstep.
  const int total = G * D;
  for (int e = tid; e < total; e += kThreads) {
    const int qc = e / D, d = e % D;
    float Mq = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mq = fmaxf(Mq, red_m[w][qc]);
    const float Mqu = (Mq == -INFINITY) ? 0.f : Mq;
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      lsum = fmaf(red_l[w][qc], exp2_fast(red_m[w][qc] - Mqu), lsum);
      osum += red_o[(w * kMaxGroup + qc) * D + d];
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int hq_out = h * G + qc;
    const int64_t row = (int64_t)b * p.Hq + hq_out;
    if (p.S == 1) {
      p.o[row * D + d] = (bf16)(osum * inv);
      if (d == 0 && p.lse != nullptr) p.lse[row] = lsum > 0.f ? (Mq + log2_fast(lsum)) * kLn2 : -INFINITY;
    } else {
      p.part_o[(row * p.S + s) * D + d] = osum * inv;
      if (d == 0) p.part_lse[row * p.S + s] = lsum > 0.f ? Mq + log2_fast(lsum) : -INFINITY;
    }
  }
}

// One wavefront per (sequence, query head): merge the splits that exist
// with weights 2^(L_s - max L) in fixed split order.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecParams p, int rows) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // b * Hq + hq
  if (row >= rows) return;
  const int b = row / p.Hq;
  const int L = seq_len(p, b);
  const int n = (L + p.chunk - 1) / p.chunk;  // splits that hold keys
  const float* pl = p.part_lse + (int64_t)row * p.S;
  float M = -INFINITY;
  for (int s = lane; s < n; s += 64) M = fmaxf(M, pl[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float Mu = (M == -INFINITY) ? 0.f : M;
  constexpr int PER = D / 64;
  float o[PER > 0 ? PER : 1] = {};
  float wsum = 0.f;
  for (int s = 0; s < n; ++s) {
    const float w = exp2_fast(pl[s] - Mu);
    wsum += w;
    const float* po = p.part_o + ((int64_t)row * p.S + s) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = fmaf(w, po[lane * PER + e], o[e]);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) p.o[(int64_t)row * D + lane * PER + e] = (bf16)(o[e] * inv);
  if (lane == 0 && p.lse != nullptr) p.lse[row] = wsum > 0.f ? (Mu + log2_fast(wsum)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  DecParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.kc = static_cast<const bf16*>(a.kcache);
  p.vc = static_cast<const bf16*>(a.vcache);
  p.lens = a.seqlens;
  p.o = static_cast<bf16*>(a.o);
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.capacity = a.capacity;
  p.S = a.num_splits;
  p.chunk = decode_chunk(a.capacity, a.num_splits);
  p.c = a.scale * kLog2e;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  if (p.S > 1) {
    p.part_o = static_cast<float*>(a.workspace);
    p.part_lse = p.part_o + (size_t)a.B * a.Hq * p.S * D;
  }
  dim3 grid(p.S, a.Hkv, a.B);
  hipLaunchKernelGGL((decode_split_kernel<D>), grid, dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  const int rows = a.B * a.Hq;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, stream, p, rows);
  return hipGetLastError();
}

}  // namespace

int decode_chunk(int capacity, int num_splits) {
  const int per = (capacity + num_splits - 1) / num_splits;
  const int c = ((per + kTile - 1) / kTile) * kTile;
  return c > 0 ? c : kTile;
}

size_t decode_workspace_bytes(int B, int Hq, int d, int num_splits) {
  if (num_splits <= 1) return 0;
  return (size_t)B * Hq * num_splits * ((size_t)d + 1) * sizeof(float);
}

bool decode_supported(int d, int group) {
  return (d == 64 || d == 128 || d == 256) && group >= 1 && group <= kMaxGroup;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch<64>(a, stream);
    case 128: return launch<128>(a, stream);
    case 256: return launch<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
