// fa_bwd.hip - backward pass (dQ, dK, dV) in bf16 for gfx950.
//
// The backward keeps only the forward's row log-sum-exp and recomputes the
// score tiles (FlashAttention: Part 2, section 1.3; the pyshine.com code
// tour describes the same recompute-then-accumulate backward). With
// P = exp(scale S - LSE) recomputed per tile, the gradients of
// O = softmax(scale Q K^T) V are
//     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_d dO_id O_id,
//     dQ = scale dS K,  dK = scale dS^T Q,
// where D_i equals sum_j P_ij dP_ij (FlashAttention: Part 2, section 1.3
// credits FA2 with trimming such non-matmul work around the softmax).
//
// Three kernels, no atomics, so the result is bitwise reproducible:
//  1. bwd_prep_kernel: D and -LSE/scale per (batch, head, query), into the
//     caller's workspace (rows padded to a multiple of 32 queries, padded
//     entries made inert: -LSE/scale = -inf gives P = 0).
//  2. bwd_dq_kernel: one workgroup per 128-query tile of one head, the
//     forward's layout (lane = query): S^T = K Q^T and dP^T = V dO^T from
//     the same LDS K/V tiles, dQ^T += K^T dS^T.
//  3. bwd_dkdv_kernel: one workgroup per 128-key tile of one key/value
//     head, lane = key: it walks every query tile of every query head of
//     the group, S = Q K^T and dP = dO V^T with K and V held in registers,
//     dV^T += dO^T P and dK^T += Q^T dS, so a grouped head's gradients sum
//     over its group inside the accumulators.
#include <stdlib.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

struct BwdParams {
  const char* __restrict__ q;
  const char* __restrict__ k;
  const char* __restrict__ v;
  const char* __restrict__ o;
  const char* __restrict__ dout;
  const float* __restrict__ lse;
  char* __restrict__ dq;
  char* __restrict__ dk;
  char* __restrict__ dv;
  float* __restrict__ dvec;  // D, (B, Hq, nq_pad), rows local to their sequence
  float* __restrict__ nlse;  // -LSE / scale, (B, Hq, nq_pad)
  int Nq, Nk, Hq, Hkv, group, B;  // dense lengths (packed batches: the longest sequences)
  int nq_pad;                // Nq rounded up to a multiple of kQStep
  float c;                   // scale * log2(e)
  float scale;
  // key j is visible to query i iff i + off - wl <= j <= i + off + wr (a
  // negative bound is unlimited), off = Nk_b - Nq_b when bottom_right,
  // else 0; top-left causal is (wl, wr) = (-1, 0)
  int wl, wr, bottom_right;
  int lpt;                   // dQ tiles longest-first (later query tiles see more keys)
  // packed variable-length batch (null: dense): sequence b is rows
  // cu_q[b] .. cu_q[b+1] of q, o, dout, dq and cu_k[b] .. cu_k[b+1] of k, v, dk, dv
  const int32_t* __restrict__ cu_q;
  const int32_t* __restrict__ cu_k;
  int total_q, total_k;      // packed row counts (LSE is then (Hq, total_q))
};

// One sequence's rows: where its queries and keys start in the (packed or
// dense) arrays, how many there are, and the window offset.
// A packed sequence longer than the launch covers (max_seqlen_q / _k) is
// `bad`: its gradient rows are all written as NaN instead.
struct Seq {
  int qrow0, Nqb, krow0, Nkb, off;
  int lq, lk;  // the sequence's own lengths
  bool bad;
};

template <bool WIN>
__device__ __forceinline__ Seq seq_of(const BwdParams& p, int b) {
  Seq s;
  if (WIN && p.cu_q != nullptr) {  // offsets clamped into the arrays
    s.qrow0 = min(max(p.cu_q[b], 0), p.total_q);
    s.lq = min(max(p.cu_q[b + 1], s.qrow0), p.total_q) - s.qrow0;
    s.Nqb = min(s.lq, p.Nq);
    s.krow0 = min(max(p.cu_k[b], 0), p.total_k);
    s.lk = min(max(p.cu_k[b + 1], s.krow0), p.total_k) - s.krow0;
    s.Nkb = min(s.lk, p.Nk);
  } else {
    s.qrow0 = b * p.Nq;
    s.Nqb = s.lq = p.Nq;
    s.krow0 = b * p.Nk;
    s.Nkb = s.lk = p.Nk;
  }
  s.bad = s.lq > p.Nq || s.lk > p.Nk;
  s.off = WIN && p.bottom_right ? s.Nkb - s.Nqb : 0;
  return s;
}

// queries per step of the dK/dV kernel (and the padding unit); 64 was
// measured to spill the single-pass kernel's 512 registers per lane
constexpr int kQStep = 32;

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO o O) and -LSE/scale
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  constexpr int TPR = D / 8;        // threads per (b, i, h) row, 8 elements each
  constexpr int RPP = 256 / TPR;    // rows per pass of the workgroup
  constexpr int U = 4;              // passes; every pass's loads are issued before any is used
  // Rows run in memory order (b, i, h) with i up to the padded length, so
  // the rows of a pass are adjacent heads of one query: contiguous bytes.
  const int part = threadIdx.x % TPR;
  const int64_t total = (int64_t)p.B * p.nq_pad * p.Hq;
  bf16x8 x[U], y[U];
  int64_t orow[U];  // (b, h, i) index of the outputs; -1 past the end
  int li_b[U], li_h[U], li_i[U];
  bool live[U];     // a row of the sequence (not padding)
  Seq sq[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t row = ((int64_t)blockIdx.x * U + u) * RPP + threadIdx.x / TPR;
    orow[u] = -1;
    live[u] = false;
    li_b[u] = li_h[u] = li_i[u] = 0;
    x[u] = y[u] = bf16x8{};
    sq[u] = Seq{0, 0, 0, 0, 0, 0, 0, false};
    if (row < total) {
      const int h = (int)(row % p.Hq);
      const int64_t bi = row / p.Hq;
      const int i = (int)(bi % p.nq_pad);
      const int b = (int)(bi / p.nq_pad);
      sq[u] = seq_of<true>(p, b);
      orow[u] = ((int64_t)b * p.Hq + h) * p.nq_pad + i;
      li_b[u] = b;
      li_h[u] = h;
      li_i[u] = i;
      if (i < sq[u].Nqb) {
        live[u] = true;
        const int64_t off = (((int64_t)sq[u].qrow0 + i) * p.Hq + h) * D * 2 + part * 16;
        x[u] = *reinterpret_cast<const bf16x8*>(p.dout + off);
        y[u] = *reinterpret_cast<const bf16x8*>(p.o + off);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)x[u][e], (float)y[u][e], acc);
#pragma unroll
    for (int w = TPR / 2; w >= 1; w /= 2) acc += __shfl_xor(acc, w, 64);
    if (orow[u] >= 0 && part == 0) {
      float nl = -INFINITY;  // padded rows: P = 0
      if (live[u]) {
        const int64_t li = p.cu_q != nullptr ? (int64_t)li_h[u] * p.total_q + sq[u].qrow0 + li_i[u]
                                              : ((int64_t)li_b[u] * p.Hq + li_h[u]) * p.Nq + li_i[u];
        const float l = p.lse[li];
        nl = l == -INFINITY ? -INFINITY : -l / p.scale;
      }
      p.dvec[orow[u]] = acc;
      p.nlse[orow[u]] = nl;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. dQ: lane = query, the forward's tiling
// ---------------------------------------------------------------------------
template <int D_, int BN_>
struct DqCfg {
  static constexpr int D = D_, BN = BN_, NW = 4, BM = 128, THREADS = 256, NST = 2;
  static constexpr int CPR = D / 8;
  static constexpr int TILE = BN * D * 2;
  static constexpr int V_REGION = NST * TILE;
  static constexpr int DMA = TILE / (THREADS * 16);
  static_assert(DMA >= 1 && TILE % (THREADS * 16) == 0 && BN % 32 == 0, "dq tile");
};

// WIN: general windows and packed batches; otherwise dense, with at most a
// top-left causal mask (window (-1, 0) or (-1, -1)), compiled without the
// general bounds
template <class C, bool WIN>
__global__ __launch_bounds__(C::THREADS, 2) void bwd_dq_kernel(BwdParams p, int n_qtiles) {
  constexpr int D = C::D, BN = C::BN, NST = C::NST, CPR = C::CPR, NBT = BN / 32;
  __shared__ __attribute__((aligned(1024))) char smem[2 * NST * C::TILE];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS3 char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int r32 = lane & 31;

  // longest-first order over (query tile, head, batch), as the forward
  const int heads = p.Hq * p.B;
  const int r = blockIdx.x / heads;
  const int rest = blockIdx.x - r * heads;
  const int pairs = p.Hkv * p.B;
  const int j = rest / pairs;
  const int pr = rest - j * pairs;
  const int b = pr / p.Hkv;
  const int kvh = pr - b * p.Hkv;
  const int hq = kvh * p.group + j;
  const int qt = p.lpt ? n_qtiles - 1 - r : r;
  const int q0 = qt * C::BM;
  const int qw0 = q0 + wave * 32;
  const Seq sq = seq_of<WIN>(p, b);
  if constexpr (WIN) {
    if (sq.bad) {  // the last query tile's workgroup also covers the rows past the grid
      fill_nan_rows<D * 2>(p.dq + (int64_t)sq.qrow0 * p.Hq * D * 2 + (int64_t)hq * D * 2, (int64_t)p.Hq * D * 2,
                           min(q0, sq.lq), qt == n_qtiles - 1 ? sq.lq : min(q0 + C::BM, sq.lq), tid, C::THREADS);
      return;
    }
  }
  if (q0 >= sq.Nqb) return;  // whole workgroup: past this sequence's queries

  const int64_t q_row = (int64_t)p.Hq * D * 2;
  const int kv_row = p.Hkv * D * 2;
  // keys some row of the tile sees: tiles t0 .. t0 + ntiles - 1
  const int q_last = min(q0 + C::BM, sq.Nqb) - 1;
  const int klo = p.wl >= 0 ? max(q0 + sq.off - p.wl, 0) : 0;
  const int khi = p.wr >= 0 ? min(q_last + sq.off + p.wr, sq.Nkb - 1) : sq.Nkb - 1;
  const int t0 = klo / BN;
  const int ntiles = khi >= klo ? khi / BN - t0 + 1 : 0;

  const char* kbase = p.k + ((int64_t)sq.krow0 * p.Hkv + kvh) * D * 2;
  const char* vbase = p.v + ((int64_t)sq.krow0 * p.Hkv + kvh) * D * 2;
  int dma_row[C::DMA], dma_col[C::DMA];
#pragma unroll
  for (int jj = 0; jj < C::DMA; ++jj) {
    const int slot = jj * C::THREADS + tid;
    dma_row[jj] = slot / CPR;
    dma_col[jj] = ((slot % CPR) ^ swz_pf<CPR>(slot / CPR)) * 16;
  }
  const uint32_t dma_lds = __builtin_amdgcn_readfirstlane(lds0 + wave * 64 * 16);
  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    const int j0 = (t0 + t) * BN;
    const char* ks = kbase + (int64_t)j0 * kv_row;
    const char* vs = vbase + (int64_t)j0 * kv_row;
    const uint32_t st = dma_lds + (uint32_t)((t % NST) * C::TILE);
    const int last = sq.Nkb - 1 - j0;  // rows past the end re-read the last key (masked later)
#pragma unroll
    for (int jj = 0; jj < C::DMA; ++jj) {
      const uint32_t off = (uint32_t)(min(dma_row[jj], last) * kv_row + dma_col[jj]);
      dma16(ks, off, st + jj * C::THREADS * 16);
      dma16(vs, off, st + C::V_REGION + jj * C::THREADS * 16);
    }
  };
  if (ntiles > 0) issue_tile(0);

  // Q^T and dO^T as B operands: register i of k-step ks = X[row][16 ks + 8 g + i]
  const int my_q = qw0 + r32;
  bf16x8 qf[D / 16], of[D / 16];
  {
    const int64_t off = ((int64_t)sq.qrow0 + my_q) * q_row + (int64_t)hq * D * 2;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = my_q < sq.Nqb ? *reinterpret_cast<const bf16x8*>(p.q + off + (ks * 16 + g * 8) * 2) : bf16x8{};
      of[ks] = my_q < sq.Nqb ? *reinterpret_cast<const bf16x8*>(p.dout + off + (ks * 16 + g * 8) * 2) : bf16x8{};
    }
  }
  const int64_t vec = ((int64_t)b * p.Hq + hq) * p.nq_pad + min(my_q, p.nq_pad - 1);
  const float cnl = p.c * p.nlse[vec];  // P = 2^(c s + cnl); -inf past Nq
  const float dval = p.dvec[vec];
  wait_vm_loads();

  // LDS read offsets: K (and V) rows as A operands (b128), K^T through the
  // transposing read, exactly as the forward reads K and V^T
  uint32_t k_off[D / 16];
  {
    const int ksw = swz_pf<CPR>(r32);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) k_off[ks] = (uint32_t)(r32 * D * 2 + (((2 * ks + g) ^ ksw) * 16));
  }
  uint32_t t_off[D / 32][2];
  {
    const int vi = lane & 15, vgrp = lane >> 4;
    const int vcol = (vgrp & 1) * 2 + ((vi & 3) >> 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * h + 4 * (vgrp >> 1) + (vi >> 2);
      const int sw = swz_pf<CPR>(row);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        t_off[dt][h] = (uint32_t)(row * D * 2 + (vi & 1) * 8 + (((4 * dt + vcol) ^ sw) * 16));
    }
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  // This wavefront's tiles (relative to t0): [t_lo, t_hi) hold a key some
  // of its rows see, [u_lo, u_hi) only keys all of its rows see (no mask).
  int t_lo = 0, t_hi = 0, u_lo = 0, u_hi = 0;
  {
    const int wq_last = min(qw0 + 31, sq.Nqb - 1);
    const int wlo = p.wl >= 0 ? max(qw0 + sq.off - p.wl, 0) : 0;
    const int whi = p.wr >= 0 ? min(wq_last + sq.off + p.wr, sq.Nkb - 1) : sq.Nkb - 1;
    if (wq_last >= qw0 && whi >= wlo) {
      t_lo = max(wlo / BN - t0, 0);
      t_hi = min(whi / BN - t0 + 1, ntiles);
      const int flo = p.wl >= 0 ? max(wq_last + sq.off - p.wl, 0) : 0;
      const int fhi = p.wr >= 0 ? min(qw0 + sq.off + p.wr, sq.Nkb - 1) : sq.Nkb - 1;
      u_lo = min(max((flo + BN - 1) / BN - t0, t_lo), t_hi);
      u_hi = min(max((fhi + 1) / BN - t0, u_lo), t_hi);
    }
  }

  auto compute_tile = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // stage base as a wave-uniform value: one add per distinct lane offset
    const uint32_t ks_base = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((t % NST) * C::TILE));
    const uint32_t vs_base = ks_base + C::V_REGION;
    f32x16 s[NBT], dp[NBT];
#pragma unroll
    for (int nb = 0; nb < NBT; ++nb) s[nb] = dp[nb] = f32x16{};
    // S^T and dP^T products n = ks NBT + nb, their K and V operands read
    // RS products ahead
    {
      constexpr int NP = (D / 16) * NBT, RS = 8;
      bf16x8 ka[NP], va[NP];
      auto rd = [&](int n) __attribute__((always_inline)) {
        const int ks = n / NBT, nb = n % NBT;
        ka[n] = *(const LDS3 bf16x8*)(uintptr_t)(ks_base + k_off[ks] + nb * 32 * D * 2);
        va[n] = *(const LDS3 bf16x8*)(uintptr_t)(vs_base + k_off[ks] + nb * 32 * D * 2);
      };
#pragma unroll
      for (int n = 0; n < RS && n < NP; ++n) rd(n);
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        if (n + RS < NP) rd(n + RS);
        const int ks = n / NBT, nb = n % NBT;
        s[nb] = mfma32x32x16(ka[n], qf[ks], s[nb]);
        dp[nb] = mfma32x32x16(va[n], of[ks], dp[nb]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (RS < NP ? RS : NP), 0);
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        if (n + RS < NP) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    }
    // dS^T = P^T o (dP^T - D), P^T = 2^(c s - c LSE / scale); key
    // j0 + 4 g + o (o = 32 nb + 8 (i/4) + i%4) is visible iff lo <= o <= hi
    bf16x8 dsf[BN / 16];
    const int jb = (t0 + t) * BN + 4 * g;
    const int lo = (p.wl >= 0 ? my_q + sq.off - p.wl : 0) - jb;
    const int hi = (p.wr >= 0 ? min(my_q + sq.off + p.wr, sq.Nkb - 1) : sq.Nkb - 1) - jb;
#pragma unroll
    for (int kk = 0; kk < BN / 16; ++kk) {
      const int nb = kk >> 1, h = (kk & 1) * 8;
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float pv = exp2_fast(fmaf(s[nb][h + i], p.c, cnl));
        if constexpr (MASK) {
          const int off = nb * 32 + 8 * ((h + i) >> 2) + ((h + i) & 3);
          if constexpr (WIN) {
            if (off < lo || off > hi) pv = 0.f;
          } else {
            if (off > hi) pv = 0.f;
          }
        }
        e[i] = pv * (dp[nb][h + i] - dval);
      }
      u32x4 w;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) w[e2] = pack_bf16x2(e[2 * e2], e[2 * e2 + 1]);
      dsf[kk] = __builtin_bit_cast(bf16x8, w);
    }
    // dQ^T += K^T dS^T, products m = dt (BN / 16) + kk, their transposed
    // K^T operands read RA products ahead; at raised issue priority, so that
    // of the two wavefronts on a SIMD one streams these MFMAs while the
    // other computes its dS (with the deeper operand reads above: 1.9%
    // faster on the causal B8 H16 N2048 backward)
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    {
      constexpr int NKK = BN / 16, NP = (D / 32) * NKK, RA = 4;
      i16x4 rt[NP][2];
      auto rd = [&](int m) __attribute__((always_inline)) {
        const int dt = m / NKK, kk = m % NKK;
        rt[m][0] = ds_read_tr(ks_base + t_off[dt][0] + kk * 16 * D * 2);
        rt[m][1] = ds_read_tr(ks_base + t_off[dt][1] + kk * 16 * D * 2);
      };
#pragma unroll
      for (int m = 0; m < RA && m < NP; ++m) rd(m);
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        if (m + RA < NP) rd(m + RA);
        const int dt = m / NKK, kk = m % NKK;
        const i16x8 vv = {rt[m][0][0], rt[m][0][1], rt[m][0][2], rt[m][0][3],
                          rt[m][1][0], rt[m][1][1], rt[m][1][2], rt[m][1][3]};
        acc[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, vv), dsf[kk], acc[dt]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (RA < NP ? RA : NP), 0);
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        if (m + RA < NP) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };

  auto sync_tile = [&](int t) __attribute__((always_inline)) {
    wait_vmcnt<0>();
    barrier();  // everyone's loads of tile t landed; tile t-1 is no longer read
    if (t + 1 < ntiles) issue_tile(t + 1);
  };
  int t = 0;
  if constexpr (WIN) {
    for (; t < t_lo; ++t) sync_tile(t);
    for (; t < u_lo; ++t) {
      sync_tile(t);
      compute_tile(t, std::true_type{});
    }
  }
  // (dense: t_lo = u_lo = 0)
  for (; t < u_hi; ++t) {
    sync_tile(t);
    compute_tile(t, std::false_type{});
  }
  for (; t < t_hi; ++t) {
    sync_tile(t);
    compute_tile(t, std::true_type{});
  }
  for (; t < ntiles; ++t) sync_tile(t);

  // dQ rows go through the idle LDS ring so that 16-byte lanes store whole
  // rows (non-temporal: written once, not read here)
  static_assert(C::NW * 32 * D * 2 <= 2 * NST * C::TILE, "dQ staging exceeds the ring");
  const uint32_t ost = lds0 + (uint32_t)(wave * 32 * D * 2);
  barrier();  // every wavefront is done reading the ring
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int c = dt * 4 + jj;  // 16-byte chunk of dims 8c .. 8c+7; half g holds 8c + 4g ..
      u32x2 w;
      w[0] = pack_bf16x2(acc[dt][4 * jj + 0] * p.scale, acc[dt][4 * jj + 1] * p.scale);
      w[1] = pack_bf16x2(acc[dt][4 * jj + 2] * p.scale, acc[dt][4 * jj + 3] * p.scale);
      *(LDS3 u32x2*)(uintptr_t)(ost + r32 * D * 2 + ((c ^ (r32 % CPR)) * 16) + g * 8) = w;
    }
  // a wavefront reads back only its own rows (its LDS instructions complete in order)
#pragma unroll
  for (int i = 0; i < 32 * CPR / 64; ++i) {
    const int slot = i * 64 + lane;
    const int rw = slot / CPR, c = slot % CPR;
    const u32x4 w = *(const LDS3 u32x4*)(uintptr_t)(ost + rw * D * 2 + ((c ^ (rw % CPR)) * 16));
    const int q = qw0 + rw;
    if (q < sq.Nqb)
      __builtin_nontemporal_store(
          w, reinterpret_cast<u32x4*>(p.dq + ((int64_t)sq.qrow0 + q) * q_row + (int64_t)hq * D * 2 + c * 16));
  }
}

// ---------------------------------------------------------------------------
// 3. dK and dV: lane = key
// ---------------------------------------------------------------------------
template <int D_, int NST_ = 2>
struct DkvCfg {
  static constexpr int D = D_, NW = 4, BK = 128, THREADS = 256, NST = NST_, BQ = kQStep, NQB = BQ / 32;
  static constexpr int CPR = D / 8;
  static constexpr int TILE = BQ * D * 2;                 // one Q (or dO) tile
  static constexpr int DO_REGION = NST * TILE;
  static constexpr int VEC_REGION = 2 * NST * TILE;       // per wave: 1 KiB per stage
  static constexpr int LDS_BYTES = VEC_REGION + NST * NW * 1024;
  static constexpr int DMA = TILE / (THREADS * 16);
  static_assert(DMA >= 1 && TILE % (THREADS * 16) == 0, "dkdv tile");
};

// WHAT selects the gradients a launch produces: kDV (S, P, dV^T += dO^T P),
// kDK (S, P, dP, dS, dK^T += Q^T dS) or both in one pass (the default: the
// split pair recomputes S once more, and although its dV half runs two
// wavefronts per SIMD, the pair measured slower than the single pass).
constexpr int kDV = 1, kDK = 2, kDKDV = 3;

template <class C, int WHAT, int WPS, bool WIN>
__global__ __launch_bounds__(C::THREADS, WPS) void bwd_dkdv_kernel(BwdParams p, int n_ktiles) {
  constexpr bool DV = (WHAT & kDV) != 0, DK = (WHAT & kDK) != 0;
  constexpr int D = C::D, NST = C::NST, CPR = C::CPR, BQ = C::BQ;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS3 char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int r32 = lane & 31;

  // (key tile, key/value head, batch); with a causal mask the first key
  // tiles see the most queries, so they go first
  const int pairs = p.Hkv * p.B;
  const int kt = blockIdx.x / pairs;
  const int pr = blockIdx.x - kt * pairs;
  const int b = pr / p.Hkv;
  const int kvh = pr - b * p.Hkv;
  const int k0 = kt * C::BK;
  const int kw0 = k0 + wave * 32;     // first key of this wavefront
  const int my_k = kw0 + r32;         // this lane's key (MFMA column)
  const Seq sq = seq_of<WIN>(p, b);
  if constexpr (WIN) {
    if (sq.bad) {  // the last key tile's workgroup also covers the rows past the grid
      const int r0 = min(k0, sq.lk), r1 = kt == n_ktiles - 1 ? sq.lk : min(k0 + C::BK, sq.lk);
      const int64_t base = (int64_t)sq.krow0 * p.Hkv * D * 2 + (int64_t)kvh * D * 2;
      if constexpr (DK) fill_nan_rows<D * 2>(p.dk + base, (int64_t)p.Hkv * D * 2, r0, r1, tid, C::THREADS);
      if constexpr (DV) fill_nan_rows<D * 2>(p.dv + base, (int64_t)p.Hkv * D * 2, r0, r1, tid, C::THREADS);
      return;
    }
  }

  const int kv_row = p.Hkv * D * 2;
  const int64_t q_row = (int64_t)p.Hq * D * 2;

  // K and V rows of this lane's key as B operands: register i of k-step ks
  // = X[key][16 ks + 8 g + i]
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int64_t off = ((int64_t)sq.krow0 + my_k) * kv_row + (int64_t)kvh * D * 2;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kf[ks] = my_k < sq.Nkb ? *reinterpret_cast<const bf16x8*>(p.k + off + (ks * 16 + g * 8) * 2) : bf16x8{};
      if constexpr (DK)
        vf[ks] = my_k < sq.Nkb ? *reinterpret_cast<const bf16x8*>(p.v + off + (ks * 16 + g * 8) * 2) : bf16x8{};
    }
  }

  // steps: query tiles of BQ rows of each query head of the group, those
  // some query of which sees a key of this workgroup: key j is seen by
  // queries j - off - wr .. j - off + wl
  int q_first = 0, per_head = 0, nsteps = 0;
  if constexpr (WIN) {
    if (k0 < sq.Nkb && sq.Nqb > 0) {
      const int k_last = min(k0 + C::BK, sq.Nkb) - 1;
      const int qlo = p.wr >= 0 ? max(k0 - sq.off - p.wr, 0) : 0;
      const int qhi = p.wl >= 0 ? min(k_last - sq.off + p.wl, sq.Nqb - 1) : sq.Nqb - 1;
      if (qhi >= qlo) {
        q_first = qlo / BQ;
        per_head = qhi / BQ - q_first + 1;
      }
    }
    nsteps = per_head * p.group;
  } else {  // top-left causal: queries below this workgroup's first key see none of it
    q_first = p.wr >= 0 ? k0 / BQ : 0;
    per_head = max((p.Nq + BQ - 1) / BQ - q_first, 0);
    nsteps = k0 < p.Nk ? per_head * p.group : 0;
  }

  int dma_row[C::DMA], dma_col[C::DMA];
#pragma unroll
  for (int jj = 0; jj < C::DMA; ++jj) {
    const int slot = jj * C::THREADS + tid;
    dma_row[jj] = slot / CPR;
    dma_col[jj] = ((slot % CPR) ^ swz_pf<CPR>(slot / CPR)) * 16;
  }
  const uint32_t dma_lds = __builtin_amdgcn_readfirstlane(lds0 + wave * 64 * 16);
  const uint32_t vec_lds = __builtin_amdgcn_readfirstlane(lds0 + C::VEC_REGION + wave * 1024);
  const uint32_t nlse_gap = (uint32_t)((const char*)p.nlse - (const char*)p.dvec);
  auto step_head = [&](int s) __attribute__((always_inline)) { return kvh * p.group + s / per_head; };
  auto step_q0 = [&](int s) __attribute__((always_inline)) { return (q_first + s % per_head) * BQ; };
  auto issue_step = [&](int s) __attribute__((always_inline)) {
    const int hq = step_head(s), q0 = step_q0(s);
    const char* qs = p.q + ((int64_t)sq.qrow0 + q0) * q_row + (int64_t)hq * D * 2;
    const char* os = p.dout + ((int64_t)sq.qrow0 + q0) * q_row + (int64_t)hq * D * 2;
    const uint32_t st = dma_lds + (uint32_t)((s % NST) * C::TILE);
    const int last = sq.Nqb - 1 - q0;  // rows past the end re-read the last query (P = 0 there)
#pragma unroll
    for (int jj = 0; jj < C::DMA; ++jj) {
      const uint32_t off = (uint32_t)(min(dma_row[jj], last) * (int)q_row + dma_col[jj]);
      dma16(qs, off, st + jj * C::THREADS * 16);
      dma16(os, off, st + C::DO_REGION + jj * C::THREADS * 16);
    }
    // -LSE/scale (lanes 0 .. BQ/4-1) and D (the next BQ/4 lanes) of the
    // step's queries, padded rows included; the other lanes repeat them.
    // The base is the D row; the -LSE/scale row sits nlse_gap bytes after it.
    const int vl = lane & (BQ / 2 - 1);
    const uint32_t voff = (vl < BQ / 4 ? nlse_gap : 0u) + 16u * (uint32_t)(vl & (BQ / 4 - 1));
    dma16(p.dvec + ((int64_t)b * p.Hq + hq) * p.nq_pad + q0, voff,
          vec_lds + (uint32_t)((s % NST) * (C::NW * 1024)));
  };
  if (nsteps > 0) issue_step(0);
  if (NST >= 3 && nsteps > 1) issue_step(1);
  wait_vm_loads();

  // LDS read offsets: Q and dO rows as A operands (b128), Q^T and dO^T
  // through the transposing read
  uint32_t a_off[D / 16];
  {
    const int ksw = swz_pf<CPR>(r32);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) a_off[ks] = (uint32_t)(r32 * D * 2 + (((2 * ks + g) ^ ksw) * 16));
  }
  uint32_t t_off[D / 32][2];
  {
    const int vi = lane & 15, vgrp = lane >> 4;
    const int vcol = (vgrp & 1) * 2 + ((vi & 3) >> 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * h + 4 * (vgrp >> 1) + (vi >> 2);
      const int sw = swz_pf<CPR>(row);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        t_off[dt][h] = (uint32_t)(row * D * 2 + (vi & 1) * 8 + (((4 * dt + vcol) ^ sw) * 16));
    }
  }

  f32x16 acck[D / 32], accv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acck[dt] = accv[dt] = f32x16{};

  // LDS stage bases as wave-uniform values: each read address is then one
  // add of a per-lane offset plus an immediate
  auto q_stage = [&](int s) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((s % NST) * C::TILE));
  };
  auto v_stage = [&](int s) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(vec_lds + (uint32_t)((s % NST) * (C::NW * 1024)));
  };

  // S and dP accumulators of step s start at -LSE/scale and -D, so that
  // after S = Q K^T and dP = dO V^T (query x key) they hold S - LSE/scale
  // and dP - D. Register i of query block qb is query m = 32 qb + 8 (i / 4)
  // + 4 g + i % 4 of the step.
  auto sdp_init = [&](int s, f32x16* sacc, f32x16* dpacc) __attribute__((always_inline)) {
    const uint32_t vs = v_stage(s);
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 nl = *(const LDS3 f32x4*)(uintptr_t)(vs + (32 * qb + 8 * q4 + 4 * g) * 4);
        const f32x4 dd = *(const LDS3 f32x4*)(uintptr_t)(vs + BQ * 4 + (32 * qb + 8 * q4 + 4 * g) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sacc[qb][4 * q4 + e] = nl[e];
          dpacc[qb][4 * q4 + e] = -dd[e];
        }
      }
  };
  // the S/dP MFMAs of a step in order j = 2 (ks NQB + qb) + (0: S, 1: dP)
  constexpr int NSDP = 2 * C::NQB * (D / 16);
  auto sdp_operand = [&](uint32_t qs, int j) __attribute__((always_inline)) {
    const int ks = (j >> 1) / C::NQB, qb = (j >> 1) % C::NQB;
    return *(const LDS3 bf16x8*)(uintptr_t)(qs + ((j & 1) ? C::DO_REGION : 0) + a_off[ks] + qb * 32 * D * 2);
  };
  auto sdp_mfma = [&](int j, const bf16x8& a, f32x16* sacc, f32x16* dpacc) __attribute__((always_inline)) {
    const int ks = (j >> 1) / C::NQB, qb = (j >> 1) % C::NQB;
    if (j & 1) {
      if constexpr (DK) dpacc[qb] = mfma32x32x16(a, vf[ks], dpacc[qb]);
    } else {
      sacc[qb] = mfma32x32x16(a, kf[ks], sacc[qb]);
    }
  };

  // P/dS of step s. Key j is visible to query i iff i + off - wl <= j <=
  // i + off + wr. With query i = q0 + c + 4 g, c the compile-time part of
  // each register, that is x_lo >= c >= ... <= x_hi below; when the step
  // needs no mask both bounds sit 2^30 keys away and never bind (sequences
  // stay below 2^30 rows), so the test is branch-free.
  struct Bounds { int x_hi, x_lo; };
  auto step_bounds = [&](int s) __attribute__((always_inline)) {
    bool masked;
    if constexpr (WIN) {
      const int q0 = step_q0(s) + sq.off;
      masked = (p.wl >= 0 && kw0 < q0 + BQ - 1 - p.wl) || (p.wr >= 0 && kw0 + 31 > q0 + p.wr);
    } else {
      masked = p.wr >= 0 && step_q0(s) < kw0 + 31;
    }
    constexpr int kFar = 1 << 30;
    const int lo = masked && p.wl >= 0 ? min(p.wl, kFar) : kFar;
    const int hi = masked && p.wr >= 0 ? min(p.wr, kFar) : kFar;
    const int qbase = step_q0(s) + (WIN ? sq.off : 0);
    const int kx = my_k - 4 * g;
    return Bounds{kx - (qbase + hi), kx - (qbase - lo)};  // invisible iff x_hi > c or x_lo < c
  };
  // element idx of the BQ x 32 / 64 P and dS values of this lane: P =
  // 2^(c (S - LSE/scale)), dS = P o (dP - D), packed by pairs into the B
  // operands pw (P) and sw (dS) over the query index
  constexpr int NE = (BQ / 16) * 8;
  auto pds_elem = [&](int idx, const f32x16* sacc, const f32x16* dpacc, Bounds bd, float& pe_prev, float& se_prev,
                      u32x4* pw, u32x4* sw) __attribute__((always_inline)) {
    const int kk = idx >> 3, i = idx & 7, qb = kk >> 1, h = (kk & 1) * 8;
    float pv = exp2_fast(sacc[qb][h + i] * p.c);
    const int c = 32 * qb + 8 * ((h + i) >> 2) + ((h + i) & 3);  // a constant after unrolling
    if (bd.x_hi > c || (WIN && bd.x_lo < c)) pv = 0.f;
    float sv = pv * dpacc[qb][h + i];
    asm volatile("" : "+v"(pv), "+v"(sv));  // computed here, not moved towards its use
    if (i & 1) {
      pw[kk][i >> 1] = pack_bf16x2(pe_prev, pv);
      sw[kk][i >> 1] = pack_bf16x2(se_prev, sv);
    } else {
      pe_prev = pv;
      se_prev = sv;
    }
  };
  // dV^T += dO^T P and dK^T += Q^T dS (d x key) for step s: products m in
  // the order (dt, kk, dV then dK), the transposed operand reads issued
  // RA products ahead so each MFMA finds its operands in registers
  auto dvdk = [&](int s, const u32x4* pw, const u32x4* sw) __attribute__((always_inline)) {
    const uint32_t qs = q_stage(s);
    const uint32_t os = qs + C::DO_REGION;
    constexpr int NKK = BQ / 16, W = (DV ? 1 : 0) + (DK ? 1 : 0), NOPS = (D / 32) * NKK * W, RA = 4;
    i16x4 rt[NOPS][2];
    auto is_dv = [&](int m) __attribute__((always_inline)) { return DV && (!DK || m % W == 0); };
    auto rd = [&](int m) __attribute__((always_inline)) {
      const int dt = m / (NKK * W), kk = (m / W) % NKK;
      const uint32_t base = is_dv(m) ? os : qs;
      rt[m][0] = ds_read_tr(base + t_off[dt][0] + kk * 16 * D * 2);
      rt[m][1] = ds_read_tr(base + t_off[dt][1] + kk * 16 * D * 2);
    };
#pragma unroll
    for (int m = 0; m < RA && m < NOPS; ++m) rd(m);
#pragma unroll
    for (int m = 0; m < NOPS; ++m) {
      if (m + RA < NOPS) rd(m + RA);
      const int dt = m / (NKK * W), kk = (m / W) % NKK;
      const i16x8 t = {rt[m][0][0], rt[m][0][1], rt[m][0][2], rt[m][0][3],
                       rt[m][1][0], rt[m][1][1], rt[m][1][2], rt[m][1][3]};
      if (is_dv(m))
        accv[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, t), __builtin_bit_cast(bf16x8, pw[kk]), accv[dt]);
      else
        acck[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, t), __builtin_bit_cast(bf16x8, sw[kk]), acck[dt]);
    }
    // issue order: the first RA products' reads, then each MFMA preceded by
    // the reads of the product RA later
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (RA < NOPS ? RA : NOPS), 0);
#pragma unroll
    for (int m = 0; m < NOPS; ++m) {
      if (m + RA < NOPS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };

  // One step's products in issue order. Step `cs` (if >= 0) has its S/dP in
  // csa/cdp: its P/dS and dV/dK are computed. Step `ns` (if >= 0) gets its
  // S/dP into nsa/ndp, each of those MFMAs followed by a share of step cs's
  // P/dS arithmetic, which the MFMA's execution then hides (one wavefront
  // per SIMD has no other wavefront to fill its matrix pipe).
  auto step_ops = [&](int cs, const f32x16* csa, const f32x16* cdp, int ns, f32x16* nsa, f32x16* ndp,
                      auto has_cur, auto has_next) __attribute__((always_inline)) {
    constexpr bool CUR = decltype(has_cur)::value, NXT = decltype(has_next)::value;
    constexpr int PF = 4;                      // operand reads ahead of their MFMA
    constexpr int EPM = (NE + NSDP - 1) / NSDP;  // P/dS elements after each MFMA
    bf16x8 opr[NSDP];
    uint32_t nqs = 0;
    if constexpr (NXT) {
      sdp_init(ns, nsa, ndp);
      nqs = q_stage(ns);
#pragma unroll
      for (int j = 0; j < PF; ++j) opr[j] = sdp_operand(nqs, j);
    }
    Bounds bd{0, 0};
    if constexpr (CUR) bd = step_bounds(cs);
    u32x4 pw[BQ / 16], sw[BQ / 16];
    float pe_prev = 0.f, se_prev = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < (NXT ? NSDP : 1); ++j) {
      if constexpr (NXT) {
        if (j + PF < NSDP) opr[j + PF] = sdp_operand(nqs, j + PF);
        sdp_mfma(j, opr[j], nsa, ndp);
      }
      if constexpr (CUR) {
#pragma unroll
        for (int e = 0; e < (NXT ? EPM : NE); ++e) {
          const int idx = (NXT ? j * EPM : 0) + e;
          if (idx < NE) pds_elem(idx, csa, cdp, bd, pe_prev, se_prev, pw, sw);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (CUR) dvdk(cs, pw, sw);
  };

  // The dK and dV accumulators stay in AGPRs across steps: without this the
  // compiler carries them in VGPRs and moves all 128 values in and out of
  // AGPRs around every step's MFMAs.
  auto pin_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      asm volatile("" : "+a"(acck[dt]));
      asm volatile("" : "+a"(accv[dt]));
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  f32x16 sa0[C::NQB], dp0[C::NQB];
  if constexpr (NST >= 3) {
    // Software pipeline over a three-stage ring: the S/dP MFMAs of step
    // s + 1 run interleaved with the P/dS arithmetic of step s. Two sets
    // of S/dP accumulators alternate between even and odd steps.
    f32x16 sa1[C::NQB], dp1[C::NQB];
    if (nsteps > 0) {
      barrier();  // everyone's loads of steps 0 and 1 landed
      step_ops(-1, sa1, dp1, 0, sa0, dp0, F_{}, T_{});
    }
    // step s with s + 1 < nsteps, PAR = s % 2
    auto pipe_step = [&](int s, auto par) __attribute__((always_inline)) {
      pin_acc();
      wait_vmcnt<0>();
      barrier();  // everyone's loads of step s + 1 landed; step s - 1 is no longer read
      if (s + 2 < nsteps) issue_step(s + 2);
      if constexpr (decltype(par)::value == 0) step_ops(s, sa0, dp0, s + 1, sa1, dp1, T_{}, T_{});
      else step_ops(s, sa1, dp1, s + 1, sa0, dp0, T_{}, T_{});
    };
    int s = 0;
    for (; s + 2 < nsteps; s += 2) {
      pipe_step(s, std::integral_constant<int, 0>{});
      pipe_step(s + 1, std::integral_constant<int, 1>{});
    }
    if (s + 1 < nsteps) {
      pipe_step(s, std::integral_constant<int, 0>{});
      ++s;
    }
    if (s < nsteps) {  // the last step: its S/dP are in the set of its parity
      pin_acc();
      if (s & 1) step_ops(s, sa1, dp1, -1, sa0, dp0, T_{}, F_{});
      else step_ops(s, sa0, dp0, -1, sa1, dp1, T_{}, F_{});
    }
  } else {
    for (int s = 0; s < nsteps; ++s) {
      pin_acc();
      wait_vmcnt<0>();
      barrier();  // everyone's loads of step s landed; step s-1 is no longer read
      if (s + 1 < nsteps) issue_step(s + 1);
      step_ops(-1, sa0, dp0, s, sa0, dp0, F_{}, T_{});
      step_ops(s, sa0, dp0, -1, sa0, dp0, T_{}, F_{});
    }
  }

  // dK and dV rows go, one after the other, through the idle LDS so that
  // 16-byte lanes store whole rows (non-temporal: written once, not read here)
  static_assert(C::NW * 32 * D * 2 <= C::LDS_BYTES, "dK/dV staging exceeds the LDS");
  const uint32_t ost = lds0 + (uint32_t)(wave * 32 * D * 2);
  auto store_rows = [&](const f32x16 (&a)[D / 32], float mul, char* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int c = dt * 4 + jj;  // 16-byte chunk of dims 8c .. 8c+7; half g holds 8c + 4g ..
        u32x2 w;
        w[0] = pack_bf16x2(a[dt][4 * jj + 0] * mul, a[dt][4 * jj + 1] * mul);
        w[1] = pack_bf16x2(a[dt][4 * jj + 2] * mul, a[dt][4 * jj + 3] * mul);
        *(LDS3 u32x2*)(uintptr_t)(ost + r32 * D * 2 + ((c ^ (r32 % CPR)) * 16) + g * 8) = w;
      }
    // a wavefront reads back only its own rows (its LDS instructions
    // complete in order, also against the next call's writes)
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int slot = i * 64 + lane;
      const int rw = slot / CPR, c = slot % CPR;
      const u32x4 w = *(const LDS3 u32x4*)(uintptr_t)(ost + rw * D * 2 + ((c ^ (rw % CPR)) * 16));
      const int k = kw0 + rw;
      if (k < sq.Nkb)
        __builtin_nontemporal_store(
            w, reinterpret_cast<u32x4*>(dst + ((int64_t)sq.krow0 + k) * kv_row + (int64_t)kvh * D * 2 + c * 16));
    }
  };
  barrier();  // every wavefront is done reading the ring
  if constexpr (DK) store_rows(acck, p.scale, p.dk);
  if constexpr (DV) store_rows(accv, 1.f, p.dv);
}

// Kernel-shape override for tuning (FA_BWD_VARIANT=1: dK and dV in two
// separate passes), read at every call.
int bwd_variant() {
  const char* e = getenv("FA_BWD_VARIANT");
  return e ? atoi(e) : 0;
}

template <int D>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const char*>(a.q);
  p.k = static_cast<const char*>(a.k);
  p.v = static_cast<const char*>(a.v);
  p.o = static_cast<const char*>(a.o);
  p.dout = static_cast<const char*>(a.dout);
  p.lse = a.lse;
  p.dq = static_cast<char*>(a.dq);
  p.dk = static_cast<char*>(a.dk);
  p.dv = static_cast<char*>(a.dv);
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.B = a.B;
  p.wl = a.window_left;
  p.wr = a.window_right;
  p.bottom_right = a.bottom_right;
  p.lpt = a.window_right >= 0;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  p.nq_pad = (a.Nq + kQStep - 1) / kQStep * kQStep;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  p.dvec = static_cast<float*>(a.workspace);
  p.nlse = p.dvec + (size_t)a.B * a.Hq * p.nq_pad;

  // the general kernels for windows other than top-left causal / none, and
  // for packed batches
  const bool win = a.cu_q != nullptr || a.bottom_right != 0 || a.window_left >= 0 ||
                   (a.window_right != 0 && a.window_right != -1);
  const int64_t rows = (int64_t)a.B * a.Hq * p.nq_pad;
  if (rows > 0) {
    constexpr int RPB = 4 * 256 / (D / 8);  // rows per workgroup: four passes
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, p);
  }
  using QC = DqCfg<D, 32>;
  const int n_qtiles = (a.Nq + QC::BM - 1) / QC::BM;
  if (n_qtiles > 0) {
    if (win)
      hipLaunchKernelGGL((bwd_dq_kernel<QC, true>), dim3(n_qtiles * a.Hq * a.B), dim3(QC::THREADS), 0, stream, p,
                         n_qtiles);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<QC, false>), dim3(n_qtiles * a.Hq * a.B), dim3(QC::THREADS), 0, stream, p,
                         n_qtiles);
  }
  using KC = DkvCfg<D>;
  const int n_ktiles = (a.Nk + KC::BK - 1) / KC::BK;
  if (n_ktiles > 0) {
    const dim3 grid(n_ktiles * a.Hkv * a.B);
    if (bwd_variant() == 1) {  // split pair: measured 9-15% slower on MI355X
      if (win) {
        hipLaunchKernelGGL((bwd_dkdv_kernel<KC, kDV, 2, true>), grid, dim3(KC::THREADS), 0, stream, p, n_ktiles);
        hipLaunchKernelGGL((bwd_dkdv_kernel<KC, kDK, 1, true>), grid, dim3(KC::THREADS), 0, stream, p, n_ktiles);
      } else {
        hipLaunchKernelGGL((bwd_dkdv_kernel<KC, kDV, 2, false>), grid, dim3(KC::THREADS), 0, stream, p, n_ktiles);
        hipLaunchKernelGGL((bwd_dkdv_kernel<KC, kDK, 1, false>), grid, dim3(KC::THREADS), 0, stream, p, n_ktiles);
      }
    } else {
      using KP = DkvCfg<D, 3>;  // pipelined: three-stage ring
      if (win)
        hipLaunchKernelGGL((bwd_dkdv_kernel<KP, kDKDV, 1, true>), grid, dim3(KP::THREADS), 0, stream, p, n_ktiles);
      else
        hipLaunchKernelGGL((bwd_dkdv_kernel<KP, kDKDV, 1, false>), grid, dim3(KP::THREADS), 0, stream, p, n_ktiles);
    }
  }
  return hipGetLastError();
}

}  // namespace

bool bwd_supported(int d) { return d == 64 || d == 128; }

size_t bwd_workspace_bytes(int B, int Hq, int Nq) {
  const size_t pad = ((size_t)Nq + kQStep - 1) / kQStep * kQStep;
  return 2 * (size_t)B * Hq * pad * sizeof(float);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch<64>(a, stream);
    case 128: return launch<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
