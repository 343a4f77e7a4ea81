// fa_fwd_f32.hip - float32 forward for gfx950 (fp32 products and sums).
//
// The same tiled online softmax as the bf16 kernel (FlashAttention: Part 2,
// section 6.2), written for the small fp32 case where accuracy, not speed,
// is the point: one thread per query row, key/value tiles staged in LDS and
// read as broadcasts, the row state (m, l, acc) in registers, normalisation
// deferred to the end (section 1.3). No bf16 rounding anywhere.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

struct F32Params {
  const float* __restrict__ q;
  const float* __restrict__ k;
  const float* __restrict__ v;
  float* __restrict__ o;
  float* __restrict__ lse;
  int Nq, Nk, Hq, Hkv, group, causal, n_qtiles;
  float c;  // scale * log2(e)
};

constexpr int kRows = 64;  // query rows per workgroup (one per thread)
constexpr int kKeys = 32;  // keys per LDS tile

template <int D>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(F32Params p) {
  __shared__ float Ks[kKeys][D];
  __shared__ float Vs[kKeys][D];
  const int tid = threadIdx.x;
  int qt = blockIdx.x;
  if (p.causal) qt = p.n_qtiles - 1 - qt;
  const int hq = blockIdx.y, b = blockIdx.z;
  const int kvh = hq / p.group;
  const int q0 = qt * kRows;
  const int my_q = q0 + tid;
  const int64_t q_stride = (int64_t)p.Hq * D, kv_stride = (int64_t)p.Hkv * D;

  float qv[D];
  float acc[D];
  {
    const float* qrow = p.q + ((int64_t)b * p.Nq + my_q) * q_stride + (int64_t)hq * D;
#pragma unroll
    for (int x = 0; x < D; ++x) {
      qv[x] = my_q < p.Nq ? qrow[x] : 0.f;
      acc[x] = 0.f;
    }
  }
  float m = -INFINITY, l = 0.f;

  int kend = p.Nk;
  if (p.causal) kend = min(kend, q0 + kRows);
  const float* kb = p.k + (int64_t)b * p.Nk * kv_stride + (int64_t)kvh * D;
  const float* vb = p.v + (int64_t)b * p.Nk * kv_stride + (int64_t)kvh * D;

  for (int j0 = 0; j0 < kend; j0 += kKeys) {
    __syncthreads();
    for (int e = tid; e < kKeys * D; e += kRows) {
      const int r = e / D, x = e % D;
      const bool ok = j0 + r < p.Nk;
      Ks[r][x] = ok ? kb[(int64_t)(j0 + r) * kv_stride + x] : 0.f;
      Vs[r][x] = ok ? vb[(int64_t)(j0 + r) * kv_stride + x] : 0.f;
    }
    __syncthreads();

    float s[kKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < kKeys; ++r) {
      float dot = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) dot = fmaf(qv[x], Ks[r][x], dot);
      const int key = j0 + r;
      const bool vis = key < p.Nk && (!p.causal || key <= my_q);
      s[r] = vis ? dot : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    const float m_new = fmaxf(m, mx * p.c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_use);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < kKeys; ++r) {
      s[r] = exp2_fast(fmaf(s[r], p.c, -m_use));
      rs += s[r];
    }
    l = fmaf(l, alpha, rs);
#pragma unroll
    for (int x = 0; x < D; ++x) {
      float a = acc[x] * alpha;
#pragma unroll
      for (int r = 0; r < kKeys; ++r) a = fmaf(s[r], Vs[r][x], a);
      acc[x] = a;
    }
  }

  if (my_q < p.Nq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = p.o + ((int64_t)b * p.Nq + my_q) * q_stride + (int64_t)hq * D;
#pragma unroll
    for (int x = 0; x < D; ++x) orow[x] = acc[x] * inv;
    if (p.lse != nullptr)
      p.lse[((int64_t)b * p.Hq + hq) * p.Nq + my_q] = l > 0.f ? (m + log2_fast(l)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  F32Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.o = static_cast<float*>(a.o);
  p.lse = a.lse;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.causal = a.causal;
  p.n_qtiles = (a.Nq + kRows - 1) / kRows;
  p.c = a.scale * kLog2e;
  dim3 grid(p.n_qtiles, a.Hq, a.B);
  hipLaunchKernelGGL((fwd_f32_kernel<D>), grid, dim3(kRows), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool fwd_f32_supported(int d) { return d == 64; }

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch<64>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
