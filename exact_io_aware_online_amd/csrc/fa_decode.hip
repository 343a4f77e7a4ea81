// fa_decode.hip - split-KV decode and log-sum-exp combine for gfx950.
//
// Decode has one query per sequence, so it streams the key/value cache and
// is bound by memory bandwidth (FlashAttention: Part 2, section 4.1). The
// cache of each sequence is cut into splits that separate workgroups load
// in parallel, and a second kernel merges their partial results
// (pyshine.com FlashAttention code tour, "Why You Need This").
//
// Split kernel: one wavefront per (split s, key/value head h, sequence b)
// serves all G = Hq / Hkv query heads that read head h, so each cache byte
// is read once. It streams its key range through a private LDS ring of
// key/value tiles (two stages of 64 keys at d = 128) filled by
// direct-to-LDS 16-byte loads with the non-temporal hint (no registers
// stage the cache, no barrier: the wavefront waits only for its own loads)
// and keeps one online-softmax state (FlashAttention: Part 2, section 6.2).
// Scores are S^T = K Q^T on the 16x16x32 bf16 MFMA with the G query heads
// as columns (the other 16 - G columns are zero); P^T then feeds
// O^T += V^T P^T from registers, the V^T operand read from the row-major V
// tile with ds_read_b64_tr_b16. The balanced form further down replaces
// the fixed splits for one query per sequence, and for several queries or
// appended rows where decode_balanced says so.
//
// Partial results: O_s (normalised, fp32) and L_s = log2 of the split's sum
// of 2^(t) in base-2 units; an empty split is never written, the combine
// derives from the sequence length which splits exist.
#include <stdlib.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

bool decode_balanced(int B, int Nq, int Hq, int Hkv, bool append);

namespace {

constexpr int kSplitAlign = 64;  // split boundaries are multiples of this many keys
constexpr int kMaxGroup = 16;    // query heads per key/value head (MFMA columns)
// growth of the row maximum (base 2) tolerated before rescaling
constexpr float kSlack = 8.f;

struct DecParams {
  const char* __restrict__ q;  // (B, Nq, Hq, D)
  char* __restrict__ kc;       // written only by the append
  char* __restrict__ vc;
  const int32_t* __restrict__ lens;
  char* __restrict__ o;          // (B, Nq, Hq, D)
  float* __restrict__ lse;       // (B, Hq, Nq)
  float* __restrict__ part_o;    // (B, Nq, Hq, S, D)
  float* __restrict__ part_lse;  // (B, Nq, Hq, S), base-2 units
  int Hq, Hkv, group, capacity, S, chunk;
  float c;  // scale * log2(e)
  // Nq queries per sequence, served as ncg groups of 16 (query, head)
  // columns; query i of sequence b is bottom-right aligned: with n = its
  // cache length plus n_new, it sees keys j <= n - Nq + i when causal
  int Nq, ncg, causal;
  // rows appended per sequence (0 or Nq): k_new / v_new (B, Nq, Hkv, D)
  // are written at rows lens[b] .. lens[b] + Nq - 1 before they are read
  int n_new;
  const char* __restrict__ kn;
  const char* __restrict__ vn;
  // paged cache (block_table non-null): sequence b's keys [i P, (i+1) P)
  // sit in page block_table[b * pages_per_seq + i] of kc / vc, each page
  // P = page_size rows of (Hkv, D); indices are clamped to [0, num_pages)
  const int32_t* __restrict__ block_table;
  int page_size, pages_per_seq, num_pages;
};

// Rows held before this call, clamped to [0, capacity].
__device__ __forceinline__ int base_len(const DecParams& p, int b) {
  return min(max(p.lens[b], 0), p.capacity);
}

// Rows attended: the held ones plus the appended ones, within capacity.
__device__ __forceinline__ int seq_len(const DecParams& p, int b) {
  return min(base_len(p, b) + p.n_new, p.capacity);
}

// Row of the (B * capacity or num_pages * page_size, Hkv, D) cache array
// that holds key `key` of sequence b.
__device__ __forceinline__ int64_t cache_row(const DecParams& p, int b, int key) {
  if (p.block_table == nullptr) return (int64_t)b * p.capacity + key;
  const int slot = key / p.page_size;
  const int page = min(max(p.block_table[(int64_t)b * p.pages_per_seq + slot], 0), p.num_pages - 1);
  return (int64_t)page * p.page_size + (key - slot * p.page_size);
}

// The same for a key that is uniform across the wavefront. The page index
// is read with a scalar load (constant address space), whose wait counts
// in lgkmcnt: a vector load's wait (vmcnt) would also drain the
// direct-to-LDS tile loads in flight.
__device__ __forceinline__ int64_t cache_row_uniform(const DecParams& p, int b, int key) {
  if (p.block_table == nullptr) return (int64_t)b * p.capacity + key;
  const int slot = __builtin_amdgcn_readfirstlane(key / p.page_size);
  const int64_t idx = (int64_t)__builtin_amdgcn_readfirstlane(b) * p.pages_per_seq + slot;
  const __attribute__((address_space(4))) int32_t* bt =
      (const __attribute__((address_space(4))) int32_t*)p.block_table;
  const int page = min(max(bt[idx], 0), p.num_pages - 1);
  return (int64_t)page * p.page_size + (key - slot * p.page_size);
}

// Tile shape: T keys per tile (a multiple of the 32-key MFMA step) and an
// NST-stage ring; one K (or V) tile is T * D * 2 bytes, moved by
// DMA = T * D * 2 / 1024 direct-to-LDS loads per lane.
template <int D, int T_, int NST_>
struct DecTile {
  static constexpr int T = T_;
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int TILE = T * D * 2;         // bytes of one K (or V) tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int DMA = TILE / 1024;        // loads per lane per tile (K or V)
  static constexpr int NST = NST_;               // ring depth
  static_assert(T % 32 == 0 && TILE % 1024 == 0 && (NST - 1) * 2 * DMA <= 63, "tile shape");
};

// One T-key tile of the decode: S^T = K Q^T on the 16x16x32 MFMA (the
// query heads of one key/value head as columns), online softmax, then
// O^T += V^T P^T, with K and V in the ring stage at LDS address `stg`.
// When MASK, key 16 tb + i of this lane is visible iff 16 tb + i <= lim.
template <int D, class TL, bool MASK>
__device__ __forceinline__ void dec_tile(f32x4 (&acc)[D / 16], float& m, float& l, const bf16x8 (&qf)[D / 32],
                                         const uint32_t (&k_off)[D / 32], const uint32_t (&v_off)[D / 16],
                                         uint32_t stg, int lim, float c) {
  constexpr int T = TL::T;
  // S^T: T keys x 16 columns, lane (col, g4) holds keys 16 tb + 4 g4 + i
  f32x4 sc[T / 16];
#pragma unroll
  for (int tb = 0; tb < T / 16; ++tb) {
    sc[tb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8 kf = *(const LDS3 bf16x8*)(uintptr_t)(stg + k_off[ks] + tb * 16 * D * 2);
      sc[tb] = mfma16x16x32(kf, qf[ks], sc[tb]);
    }
  }
  if constexpr (MASK) {
#pragma unroll
    for (int tb = 0; tb < T / 16; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * tb + i > lim) sc[tb][i] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int tb = 0; tb < T / 16; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[tb][i]);
  mx = quarters_max(mx);
  const float m_cand = fmaxf(m, mx * c);
  // move the reference max only when it grew by more than kSlack (see the
  // prefill kernel: O = acc / l does not depend on the reference)
  const bool rescale = __builtin_amdgcn_ballot_w64(m_cand > m + kSlack) != 0;
  float alpha = 1.f;
  if (rescale) {
    const float mu = (m_cand == -INFINITY) ? 0.f : m_cand;
    alpha = exp2_fast(m - mu);
    l *= alpha;
    m = m_cand;
  }
  const float m_use = (m == -INFINITY) ? 0.f : m;
  float rs = 0.f;
#pragma unroll
  for (int tb = 0; tb < T / 16; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[tb][i] = exp2_fast(fmaf(sc[tb][i], c, -m_use));
      rs += sc[tb][i];
    }
  l += rs;
  // branch-free (alpha is 1 when nothing moved): keeps the accumulator's
  // loop-carried registers free of conditional copies
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] *= alpha;
  // O^T += V^T P^T over 32-key steps: registers 0..3 hold keys 32 kk + 4 g4 + r,
  // 4..7 keys 32 kk + 16 + 4 g4 + r
#pragma unroll
  for (int kk = 0; kk < T / 32; ++kk) {
    u32x4 w;
    w[0] = pack_bf16x2(sc[2 * kk][0], sc[2 * kk][1]);
    w[1] = pack_bf16x2(sc[2 * kk][2], sc[2 * kk][3]);
    w[2] = pack_bf16x2(sc[2 * kk + 1][0], sc[2 * kk + 1][1]);
    w[3] = pack_bf16x2(sc[2 * kk + 1][2], sc[2 * kk + 1][3]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const i16x4 v0 = ds_read_tr(stg + v_off[dt] + kk * 32 * D * 2);
      const i16x4 v1 = ds_read_tr(stg + v_off[dt] + (kk * 32 + 16) * D * 2);
      const i16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      acc[dt] = mfma16x16x32(__builtin_bit_cast(bf16x8, vv), pf, acc[dt]);
    }
  }
}

// One wavefront per (split, key/value head, sequence). The wavefront keeps
// an NST-stage LDS ring of K/V tiles filled by direct-to-LDS loads and needs
// no barrier: it waits for its own loads (vmcnt) before reading a stage.
template <int D, class TL>
__global__ __launch_bounds__(64, 2) void decode_split_kernel(DecParams p) {
  constexpr int T = TL::T, CPR = TL::CPR, NST = TL::NST;
  __shared__ __attribute__((aligned(1024))) char smem[NST * TL::STAGE];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS3 char*)smem;

  const int lane = threadIdx.x;
  const int col = lane & 15;  // MFMA column: one (query, query head) pair
  const int g4 = lane >> 4;   // lane quarter
  // The Hkv heads of one (sequence, split) are adjacent in dispatch order,
  // so together they stream whole contiguous cache rows. Splits go in
  // decreasing index: the last splits exist only for the longest sequences
  // (or are empty and exit at once), so the tail of the launch is made of
  // split 0 .. 1 workgroups, present and full-length for every sequence.
  const int h = (int)blockIdx.x / p.ncg, cg = (int)blockIdx.x - h * p.ncg;
  const int b = blockIdx.y, s = p.S - 1 - (int)blockIdx.z;
  const int base = base_len(p, b);
  const int L = seq_len(p, b);
  const int start = s * p.chunk;
  const int end = min(start + p.chunk, L);
  if (start >= end && !(p.S == 1 && start == 0)) return;  // empty split: nothing to write
  const int ntiles = end > start ? (end - start + T - 1) / T : 0;

  const int G = p.group;
  const int kv_row = p.Hkv * D * 2;  // bytes between cache rows

  // Append: this split's share [max(start, base), end) of the new rows goes
  // into the cache before any of it is read back. Every column group of
  // the split writes the same bytes; each reads only after its own writes
  // have completed, so all of them see the new rows.
  if (p.n_new > 0 && end > max(start, base)) {
    const int r0 = max(start, base);
    for (int idx = lane; idx < (end - r0) * TL::CPR; idx += 64) {
      const int r = r0 + idx / TL::CPR, cc = idx % TL::CPR;
      const int64_t src = (((int64_t)b * p.Nq + (r - base)) * p.Hkv + h) * D * 2 + cc * 16;
      const int64_t dst = (cache_row(p, b, r) * p.Hkv + h) * D * 2 + cc * 16;
      *reinterpret_cast<u32x4*>(p.kc + dst) = *reinterpret_cast<const u32x4*>(p.kn + src);
      *reinterpret_cast<u32x4*>(p.vc + dst) = *reinterpret_cast<const u32x4*>(p.vn + src);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    wait_vm_loads();
  }

  // Column col of group cg: query qi = c / G, head g = c % G (c = 16 cg + col).
  // Its last visible key, relative to the split start, bounds the mask.
  const int cidx = 16 * cg + col;
  const bool cvalid = cidx < p.Nq * G;
  const int qi = cvalid ? cidx / G : p.Nq - 1;
  const int n_all = base + p.n_new;  // causal alignment point (may pass capacity)
  const int climit = (p.causal ? min(end - 1, n_all - p.Nq + qi) : end - 1) - start;
  // tiles whose every key is visible to every column of the group
  const int first_q = min(16 * cg / G, p.Nq - 1);
  const int gmin = (p.causal ? min(end - 1, n_all - p.Nq + first_q) : end - 1) - start;
  const int nfull = max(gmin + 1, 0) / T;

  // DMA addressing: load j of a tile fills slot 64 j + lane (row slot / CPR)
  int dma_row[TL::DMA], dma_col[TL::DMA];
#pragma unroll
  for (int j = 0; j < TL::DMA; ++j) {
    const int slot = j * 64 + lane;
    dma_row[j] = slot / CPR;
    dma_col[j] = ((slot % CPR) ^ swz<CPR>(slot / CPR)) * 16;
  }
  auto issue_tile = [&](int t) {
    const int j0 = t * T;
    const int last = end - start - 1 - j0;  // rows past the end re-read the last key (masked later)
    // a tile never straddles pages: page_size and the split starts are
    // multiples of the 64-key split alignment, tiles divide it
    const int64_t row = cache_row_uniform(p, b, start + j0);
    const char* ks = p.kc + (row * p.Hkv + h) * D * 2;
    const char* vs = p.vc + (row * p.Hkv + h) * D * 2;
    const uint32_t st = lds0 + (uint32_t)((t % NST) * TL::STAGE);
#pragma unroll
    for (int j = 0; j < TL::DMA; ++j)
      dma16<true>(ks, (uint32_t)(min(dma_row[j], last) * kv_row + dma_col[j]), st + j * 1024);
#pragma unroll
    for (int j = 0; j < TL::DMA; ++j)
      dma16<true>(vs, (uint32_t)(min(dma_row[j], last) * kv_row + dma_col[j]), st + TL::TILE + j * 1024);
  };
#pragma unroll
  for (int t = 0; t < NST - 1; ++t)
    if (t < ntiles) issue_tile(t);

  // Q^T as B operand of 16x16x32: register i of k-step ks = Q[qi][h G + g][32 ks + 8 g4 + i]
  const int hq = h * G + (cvalid ? cidx - qi * G : 0);
  const int64_t orow = ((int64_t)b * p.Nq + qi) * p.Hq + hq;  // row of o and of the partials
  bf16x8 qf[D / 32];
  {
    const char* qrow = p.q + orow * D * 2;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[ks] = cvalid ? *reinterpret_cast<const bf16x8*>(qrow + (ks * 32 + g4 * 8) * 2) : bf16x8{};
  }
  wait_vm_loads();

  // per-lane LDS offsets within a stage
  uint32_t k_off[D / 32];
  {
    const int sw = swz<CPR>(col);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) k_off[ks] = (uint32_t)(col * D * 2 + (((4 * ks + g4) ^ sw) * 16));
  }
  uint32_t v_off[D / 16];
  {
    const int row = 4 * g4 + (col >> 2);
    const int sw = swz<CPR>(row);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      v_off[dt] = (uint32_t)(TL::TILE + row * D * 2 + (col & 1) * 8 + (((2 * dt + ((col & 3) >> 1)) ^ sw) * 16));
  }

  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{};
  float m = -INFINITY, l = 0.f;

  auto compute_tile = [&](int t, auto mask_tag) {
    dec_tile<D, TL, decltype(mask_tag)::value>(acc, m, l, qf, k_off, v_off, lds0 + (uint32_t)((t % NST) * TL::STAGE),
                                               climit - t * T - 4 * g4, p.c);
  };

  auto wait_tile = [&](int t) {
    // loads issued after tile t: tiles t+1 .. min(t+NST-1, ntiles-1)
    const int after = min(NST - 1, ntiles - 1 - t);
    if (after >= 3) wait_vmcnt<(NST >= 4 ? 6 * TL::DMA : 0)>();
    else if (after == 2) wait_vmcnt<(NST >= 3 ? 4 * TL::DMA : 0)>();
    else if (after == 1) wait_vmcnt<2 * TL::DMA>();
    else wait_vmcnt<0>();
  };

  int t = 0;
  for (; t < min(nfull, ntiles); ++t) {
    if (t + NST - 1 < ntiles) issue_tile(t + NST - 1);
    wait_tile(t);
    compute_tile(t, std::false_type{});
  }
  for (; t < ntiles; ++t) {
    if (t + NST - 1 < ntiles) issue_tile(t + NST - 1);
    wait_tile(t);
    compute_tile(t, std::true_type{});
  }

  // epilogue: sum l over the lane quarters, normalise, write
  l = quarters_sum(l);
  if (cvalid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t row = orow;
    if (p.S == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
        w[1] = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
        *reinterpret_cast<u32x2*>(p.o + (row * D + dt * 16 + 4 * g4) * 2) = w;
      }
      if (g4 == 0 && p.lse != nullptr)
        p.lse[((int64_t)b * p.Hq + hq) * p.Nq + qi] = l > 0.f ? (m + log2_fast(l)) * kLn2 : -INFINITY;
    } else {
      float* po = p.part_o + (row * p.S + s) * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        *reinterpret_cast<f32x4*>(po + dt * 16 + 4 * g4) = acc[dt] * inv;
      if (g4 == 0) p.part_lse[row * p.S + s] = l > 0.f ? m + log2_fast(l) : -INFINITY;
    }
  }
}

// One wavefront per (sequence, query head): merge the splits that exist
// with weights 2^(L_s - max L) in fixed split order.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecParams p, int rows) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * Nq + i) * Hq + hq
  if (row >= rows) return;
  const int bi = row / p.Hq, hq = row - bi * p.Hq;
  const int b = bi / p.Nq, qi = bi - b * p.Nq;
  const int L = seq_len(p, b);
  const int n = (L + p.chunk - 1) / p.chunk;  // splits that hold keys
  const float* pl = p.part_lse + (int64_t)row * p.S;
  constexpr int PER = D / 64;
  // U splits at a time: every partial of a group is loaded before any is
  // used, so a group costs one memory latency rather than U; indices past
  // the last split re-read it and are not summed. The sums run in split order.
  constexpr int U = 8;
  float ls[U], po[U][PER];
  auto load_group = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + u, n - 1);
      ls[u] = pl[s];
      const float* src = p.part_o + ((int64_t)row * p.S + s) * D + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) po[u][e] = src[e];
    }
  };
  float o[PER] = {};
  float wsum = 0.f;
  auto add_group = [&](int s0, float Mu) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < n) {
        const float w = exp2_fast(ls[u] - Mu);
        wsum += w;
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = fmaf(w, po[u][e], o[e]);
      }
    }
  };
  float M = -INFINITY;
  if (n <= U) {
    // the common case: one group, whose log-sum-exps give the maximum
    if (n > 0) load_group(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u < n) M = fmaxf(M, ls[u]);
  } else {
    for (int s = lane; s < n; s += 64) M = fmaxf(M, pl[s]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  }
  const float Mu = (M == -INFINITY) ? 0.f : M;
  if (n <= U) {
    if (n > 0) add_group(0, Mu);
  } else {
    for (int s0 = 0; s0 < n; s0 += U) {
      load_group(s0);
      add_group(s0, Mu);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) reinterpret_cast<bf16*>(p.o)[(int64_t)row * D + lane * PER + e] = (bf16)(o[e] * inv);
  if (lane == 0 && p.lse != nullptr)
    p.lse[((int64_t)b * p.Hq + hq) * p.Nq + qi] = wsum > 0.f ? (Mu + log2_fast(wsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Balanced split, for calls whose queries of one sequence and key/value
// head fit one group of 16 MFMA columns (Nq G <= 16, column qi G + g for
// query qi and head h G + g), appended rows included. The cache work is
// the list of tiles of every (sequence b, key/value head h) pair, in that
// order: pair (b, h) holds n_b = ceil(L_b / T) tiles (L_b the held plus the
// appended rows, within capacity), at flat positions
// Hkv P(b) + h n_b .. + n_b - 1 with P(b) = n_0 + .. + n_(b-1). The U
// units of the launch take equal runs of it: unit u covers flat tiles
// [floor(u A / U), floor((u+1) A / U)), A the total, so every wavefront
// streams the same number of cache bytes whatever the lengths (the split
// of the cache over thread blocks that the pyshine.com code tour, "Why You
// Need This", describes for decode, with its pieces cut by work rather
// than by position). A unit writes one partial (O, LSE) per column of each
// pair its run touches, at slot u + Hkv NZ(b) + h (NZ(b) = sequences
// before b that hold keys); the slots of one pair are consecutive, and the
// combine kernel finds them from the same prefix sums. The unit whose run
// holds a tile that appended rows fall in writes them into the cache just
// before it loads that tile, so every tile is written and read by one
// wavefront.
// ---------------------------------------------------------------------------

// Rows a pair attends, held plus appended within capacity, for a held
// length `len` as read from the lengths array. MQ: the call may have
// several queries per sequence or appended rows; the one-query form is
// compiled apart so that it carries none of their work.
template <bool MQ>
__device__ __forceinline__ int lean_rows(const DecParams& p, int len) {
  if constexpr (MQ) return min(min(max(len, 0), p.capacity) + p.n_new, p.capacity);
  return min(max(len, 0), p.capacity);
}

// Held length of sequence b by a scalar load (uniform b).
__device__ __forceinline__ int lean_len_uniform(const DecParams& p, int b) {
  const __attribute__((address_space(4))) int32_t* lens =
      (const __attribute__((address_space(4))) int32_t*)p.lens;
  return lens[b];
}

// Tiles of sequence b per key/value head.
template <int T, bool MQ>
__device__ __forceinline__ int lean_tiles_uniform(const DecParams& p, int b) {
  return (lean_rows<MQ>(p, lean_len_uniform(p, b)) + T - 1) / T;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Sum over all sequences of n_b (per key/value head), by one wavefront.
template <int T, bool MQ>
__device__ __forceinline__ int64_t lean_total(const DecParams& p, int B, int lane) {
  int64_t tot = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    int n = b < B ? (lean_rows<MQ>(p, p.lens[b]) + T - 1) / T : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) n += __shfl_xor(n, off, 64);
    tot += n;
  }
  return tot;
}

// The sequence holding flat tile `target` (< Hkv * total): b, n_b, P(b) and
// NZ(b), wave-uniform.
struct LeanSeq {
  int b, nb;
  int64_t pre;  // P(b)
  int nz;       // NZ(b)
};
template <int T, bool MQ>
__device__ __forceinline__ LeanSeq lean_locate(const DecParams& p, int B, int64_t target, int lane) {
  int64_t pre = 0;
  int nz = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int n = b < B ? (lean_rows<MQ>(p, p.lens[b]) + T - 1) / T : 0;
    const int incl = wave_incl_scan(n, lane);
    const int nzi = wave_incl_scan(n > 0 ? 1 : 0, lane);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(b < B && (int64_t)p.Hkv * (pre + incl) > target);
    if (hit != 0) {
      const int j = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
      LeanSeq r;
      r.b = b0 + j;
      r.nb = __builtin_amdgcn_readfirstlane(__shfl(n, j, 64));
      const int64_t pr = pre + __shfl(incl, j, 64) - r.nb;
      r.pre = (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)pr) |
              ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)pr >> 32)) << 32);
      r.nz = __builtin_amdgcn_readfirstlane(nz + __shfl(nzi, j, 64) - (r.nb > 0 ? 1 : 0));
      return r;
    }
    pre += __shfl(incl, 63, 64);
    nz += __shfl(nzi, 63, 64);
  }
  return LeanSeq{B, 0, pre, nz};  // not reached for target < Hkv * total
}

// unit of flat tile t: the largest u with floor(u A / U) <= t
__device__ __forceinline__ int64_t lean_unit_of(int64_t t, int64_t A, int64_t U) {
  return ((t + 1) * U - 1) / A;
}

template <int D, class TL, bool MQ>
__global__ __launch_bounds__(64, 2) void decode_lean_kernel(DecParams p, int B, int64_t U) {
  constexpr int T = TL::T, CPR = TL::CPR;
  static_assert(TL::NST == 2, "the lean decode keeps one tile in flight");
  constexpr int QBYTES = kMaxGroup * D * 2;  // room for the largest group's query rows
  __shared__ __attribute__((aligned(1024))) char smem[2 * TL::STAGE + 2 * QBYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS3 char*)smem;
  const uint32_t qlds = lds0 + 2 * TL::STAGE;

  const int lane = threadIdx.x;
  const int col = lane & 15;  // MFMA column: query qi = col / G, query head h G + col % G
  const int g4 = lane >> 4;
  const int G = p.group;
  const int C = MQ ? p.Nq * G : G;  // columns in use (at most 16)
  const int Hkv = p.Hkv;
  const int64_t u = blockIdx.x;

  const int64_t A = (int64_t)Hkv * lean_total<T, MQ>(p, B, lane);
  if (A == 0) return;
  // run [t0, t1) of this unit; A = q U + r keeps the products in range
  const int64_t qa = A / U, ra = A % U;
  const int64_t t0 = qa * u + (ra * u) / U;
  const int64_t t1 = qa * (u + 1) + (ra * (u + 1)) / U;
  if (t0 >= t1) return;
  const int count = (int)(t1 - t0);

  // cursor: tile i of pair (b, h); nb = n_b, nz = NZ(b)
  struct Cur {
    int b, h, i, nb, nz;
  };
  Cur cc;
  {
    const LeanSeq sq = lean_locate<T, MQ>(p, B, t0, lane);
    const int64_t r = t0 - (int64_t)Hkv * sq.pre;
    cc.b = sq.b;
    cc.nb = sq.nb;
    cc.nz = sq.nz;
    cc.h = (int)(r / sq.nb);
    cc.i = (int)(r - (int64_t)cc.h * sq.nb);
  }
  wait_vm_loads();  // the lengths read above have landed before the tile loads start
  auto advance = [&](Cur& c) {
    if (++c.i < c.nb) return;
    c.i = 0;
    if (++c.h < Hkv) return;
    c.h = 0;
    c.nz += 1;
    do {
      ++c.b;
      c.nb = c.b < B ? lean_tiles_uniform<T, MQ>(p, c.b) : 1;
    } while (c.nb == 0);
  };

  const int kv_row = Hkv * D * 2;
  constexpr int QD = (QBYTES + 1023) / 1024;  // at most this many 16-byte loads per lane for the query rows
  const int qbytes = C * D * 2;
  const int qd = (qbytes + 1023) / 1024;
  // byte offset of this lane's 16-byte piece j of a pair's query rows (column
  // by column, D * 2 bytes each) from query 0, head h G of its sequence
  auto q_off = [&](int j) {
    const int x = min((j * 64 + lane) * 16, qbytes - 16);
    if constexpr (!MQ) return (uint32_t)x;  // one query: the G rows are contiguous
    const int cl = x / (D * 2), qq = cl / G;
    return (uint32_t)(((qq * p.Hq + (cl - qq * G)) * D * 2) + (x - cl * D * 2));
  };
  int dma_row[TL::DMA], dma_col[TL::DMA];
#pragma unroll
  for (int j = 0; j < TL::DMA; ++j) {
    const int slot = j * 64 + lane;
    dma_row[j] = slot / CPR;
    dma_col[j] = ((slot % CPR) ^ swz<CPR>(slot / CPR)) * 16;
  }
  // tile k of the run (cursor c) into stage k % 2; a tile that starts a
  // pair is preceded by the pair's query rows (C x D) into query buffer
  // `qb`, and a tile that appended rows fall in by their cache writes
  auto issue = [&](const Cur& c, int k, int qb) {
    if (c.i == 0 || k == 0) {
      const char* qs = p.q + ((int64_t)c.b * p.Nq * p.Hq + (int64_t)c.h * G) * D * 2;
#pragma unroll
      for (int j = 0; j < QD; ++j)
        if (j < qd) dma16(qs, q_off(j), qlds + qb * QBYTES + j * 1024);
    }
    if (MQ && p.n_new > 0) {
      const int base = min(max(lean_len_uniform(p, c.b), 0), p.capacity);
      const int r0 = max(c.i * T, base), r1 = min((c.i + 1) * T, min(base + p.n_new, p.capacity));
      if (r0 < r1) {
        for (int idx = lane; idx < (r1 - r0) * CPR; idx += 64) {
          const int r = r0 + idx / CPR, ch = idx % CPR;
          const int64_t src = (((int64_t)c.b * p.Nq + (r - base)) * Hkv + c.h) * D * 2 + ch * 16;
          const int64_t dst = (cache_row(p, c.b, r) * Hkv + c.h) * D * 2 + ch * 16;
          *reinterpret_cast<u32x4*>(p.kc + dst) = *reinterpret_cast<const u32x4*>(p.kn + src);
          *reinterpret_cast<u32x4*>(p.vc + dst) = *reinterpret_cast<const u32x4*>(p.vn + src);
        }
        // the rows are in memory before this wavefront's tile loads read them
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    }
    const int len = c.i == c.nb - 1 ? lean_rows<MQ>(p, lean_len_uniform(p, c.b)) : (c.i + 1) * T;
    const int last = len - 1 - c.i * T;  // rows past the end re-read the last key (masked later)
    const int64_t row = cache_row_uniform(p, c.b, c.i * T);
    const char* ks = p.kc + (row * Hkv + c.h) * D * 2;
    const char* vs = p.vc + (row * Hkv + c.h) * D * 2;
    const uint32_t st = lds0 + (uint32_t)((k & 1) * TL::STAGE);
#pragma unroll
    for (int j = 0; j < TL::DMA; ++j)
      dma16<true>(ks, (uint32_t)(min(dma_row[j], last) * kv_row + dma_col[j]), st + j * 1024);
#pragma unroll
    for (int j = 0; j < TL::DMA; ++j)
      dma16<true>(vs, (uint32_t)(min(dma_row[j], last) * kv_row + dma_col[j]), st + TL::TILE + j * 1024);
  };

  uint32_t k_off[D / 32];
  {
    const int sw = swz<CPR>(col);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) k_off[ks] = (uint32_t)(col * D * 2 + (((4 * ks + g4) ^ sw) * 16));
  }
  uint32_t v_off[D / 16];
  {
    const int row = 4 * g4 + (col >> 2);
    const int sw = swz<CPR>(row);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      v_off[dt] = (uint32_t)(TL::TILE + row * D * 2 + (col & 1) * 8 + (((2 * dt + ((col & 3) >> 1)) ^ sw) * 16));
  }

  bf16x8 qf[D / 32];
  f32x4 acc[D / 16];
  float m = -INFINITY, l = 0.f;
  const bool cvalid = col < C;
  const int qi = MQ && cvalid ? col / G : (MQ ? p.Nq - 1 : 0);
  // last key this lane's column sees in the pair being computed, and the
  // smallest such key over the columns (tiles past it are masked)
  int lastkey = 0, minkey = 0;
  int qbuf = 0;  // query buffer of the pair being computed

  Cur ic = cc;  // issue cursor, one tile ahead
  issue(ic, 0, 0);
  int ibuf = 0;  // query buffer of the pair the issue cursor is in
  for (int k = 0; k < count; ++k) {
    bool next_new = false;
    if (k + 1 < count) {
      advance(ic);
      next_new = ic.i == 0;
      if (next_new) ibuf ^= 1;
      issue(ic, k + 1, ibuf);
    }
    // tile k (and its pair's query rows) landed: at most tile k + 1's loads remain
    if (k + 1 < count) {
      if (next_new) {
        static_for<QD + 1>([&](auto Q) {
          if (qd == decltype(Q)::value) wait_vmcnt<2 * TL::DMA + decltype(Q)::value>();
        });
      } else {
        wait_vmcnt<2 * TL::DMA>();
      }
    } else {
      wait_vmcnt<0>();
    }
    const bool seg_start = k == 0 || cc.i == 0;
    if (seg_start) {
      // this pair's query rows: column col is query qi, query head h G + col - qi G
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const bf16x8 x = *(const LDS3 bf16x8*)(uintptr_t)(qlds + qbuf * QBYTES + (col * D + ks * 32 + g4 * 8) * 2);
        qf[ks] = cvalid ? x : bf16x8{};
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{};
      m = -INFINITY;
      l = 0.f;
      if constexpr (MQ) {
        // query qi is bottom-right aligned with the held and appended rows:
        // with causal masking it sees keys j <= held + appended - Nq + qi
        const int held = lean_len_uniform(p, cc.b);
        const int len = lean_rows<MQ>(p, held);
        const int n_all = min(max(held, 0), p.capacity) + p.n_new;
        lastkey = p.causal ? min(len - 1, n_all - p.Nq + qi) : len - 1;
        minkey = p.causal ? min(len - 1, n_all - p.Nq) : len - 1;
      }
    }
    const uint32_t stg = lds0 + (uint32_t)((k & 1) * TL::STAGE);
    const bool last_of_pair = cc.i == cc.nb - 1;
    if (!MQ && last_of_pair) {
      const int len = lean_rows<MQ>(p, lean_len_uniform(p, cc.b));
      dec_tile<D, TL, true>(acc, m, l, qf, k_off, v_off, stg, len - 1 - cc.i * T - 4 * g4, p.c);
    } else if (MQ && (last_of_pair || (cc.i + 1) * T - 1 > minkey)) {
      dec_tile<D, TL, true>(acc, m, l, qf, k_off, v_off, stg, lastkey - cc.i * T - 4 * g4, p.c);
    } else {
      dec_tile<D, TL, false>(acc, m, l, qf, k_off, v_off, stg, 0, p.c);
    }
    if (last_of_pair || k + 1 == count) {
      // this run's part of the pair: normalised O and base-2 LSE
      const float lt = quarters_sum(l);
      const int64_t slot = u + (int64_t)Hkv * cc.nz + cc.h;
      if (cvalid) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        float* po = p.part_o + (slot * C + col) * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16 + 4 * g4) = acc[dt] * inv;
        if (g4 == 0) p.part_lse[slot * C + col] = lt > 0.f ? m + log2_fast(lt) : -INFINITY;
      }
    }
    // the query buffer a new pair's rows went into
    const bool next_starts = k + 1 < count && last_of_pair;
    advance(cc);
    if (next_starts) qbuf ^= 1;
  }
}

// One wavefront per (sequence, query, query head): merge the parts of its
// pair's column in unit order with weights 2^(L_s - max L).
template <int D, int T, bool MQ>
__global__ __launch_bounds__(256) void decode_lean_combine_kernel(DecParams p, int B, int64_t U) {
  const int lane = threadIdx.x & 63;
  const int Nq = MQ ? p.Nq : 1;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // (b Nq + qi) Hq + hq: the row of o
  if (row >= B * Nq * p.Hq) return;
  const int b = row / (Nq * p.Hq), qh = row - b * Nq * p.Hq;
  const int qi = MQ ? qh / p.Hq : 0, hq = qh - qi * p.Hq;
  const int G = p.group;
  const int C = Nq * G;
  const int h = hq / G, g = qi * G + (hq - h * G);  // g: the column
  const int64_t A = (int64_t)p.Hkv * lean_total<T, MQ>(p, B, lane);
  // P(b), n_b and NZ(b) from the same scan the units used
  int64_t pre = 0;
  int nz = 0, nb = 0;
  for (int b0 = 0; b0 <= b; b0 += 64) {
    const int bb = b0 + lane;
    const int n = bb < B ? (lean_rows<MQ>(p, p.lens[bb]) + T - 1) / T : 0;
    const int incl = wave_incl_scan(bb < b ? n : 0, lane);
    const int nzi = wave_incl_scan(bb < b && n > 0 ? 1 : 0, lane);
    if (b < b0 + 64) nb = __shfl(n, b - b0, 64);
    pre += __shfl(incl, 63, 64);
    nz += __shfl(nzi, 63, 64);
  }
  constexpr int PER = D / 64;
  float o[PER] = {};
  float wsum = 0.f, M = -INFINITY;  // running maximum of the merged L_s
  if (nb > 0) {
    const int64_t s0 = (int64_t)p.Hkv * pre + (int64_t)h * nb;
    const int64_t u0 = lean_unit_of(s0, A, U), u1 = lean_unit_of(s0 + nb - 1, A, U);
    const int64_t slot0 = u0 + (int64_t)p.Hkv * nz + h;
    const int n = (int)(u1 - u0 + 1);
    const float* pl = p.part_lse + slot0 * C + g;
    // with more units than tiles some units own no tile and write nothing:
    // their slots are skipped (unit u's run is empty iff its start equals
    // the next unit's)
    const int64_t qa = A / U, ra = A % U;
    auto unit_start = [&](int64_t uu) { return qa * uu + (ra * uu) / U; };
    auto has_part = [&](int s) { return A >= U || unit_start(u0 + s) < unit_start(u0 + s + 1); };
    // UG parts at a time, all loaded before any is used, merged in unit
    // order against a running maximum (one round of loads for the usual
    // two or three parts)
    constexpr int UG = 8;
    for (int s0p = 0; s0p < n; s0p += UG) {
      float ls[UG], po[UG][PER];
#pragma unroll
      for (int uu = 0; uu < UG; ++uu) {
        const int s = min(s0p + uu, n - 1);
        ls[uu] = pl[(int64_t)s * C];
        const float* src = p.part_o + ((slot0 + s) * C + g) * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) po[uu][e] = src[e];
      }
      // which of the UG slots hold a part: lane j answers for slot s0p + j
      const uint64_t held = __builtin_amdgcn_ballot_w64(lane < UG && s0p + lane < n && has_part(s0p + lane));
#pragma unroll
      for (int uu = 0; uu < UG; ++uu)
        if (((held >> uu) & 1) == 0) ls[uu] = -INFINITY;
      float cm = M;
#pragma unroll
      for (int uu = 0; uu < UG; ++uu) cm = fmaxf(cm, ls[uu]);
      if (cm == -INFINITY) continue;  // nothing with keys yet
      const float r = exp2_fast(M - cm);  // 0 while M is -inf
      wsum *= r;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] *= r;
#pragma unroll
      for (int uu = 0; uu < UG; ++uu) {
        if (ls[uu] != -INFINITY) {
          const float w = exp2_fast(ls[uu] - cm);
          wsum += w;
#pragma unroll
          for (int e = 0; e < PER; ++e) o[e] = fmaf(w, po[uu][e], o[e]);
        }
      }
      M = cm;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) reinterpret_cast<bf16*>(p.o)[(int64_t)row * D + lane * PER + e] = (bf16)(o[e] * inv);
  if (lane == 0 && p.lse != nullptr)
    p.lse[MQ ? ((int64_t)b * p.Hq + hq) * Nq + qi : (int64_t)row] = wsum > 0.f ? (M + log2_fast(wsum)) * kLn2
                                                                           : -INFINITY;
}

template <int D, class TL>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  DecParams p;
  p.q = static_cast<const char*>(a.q);
  p.kc = static_cast<char*>(const_cast<void*>(a.kcache));
  p.vc = static_cast<char*>(const_cast<void*>(a.vcache));
  p.lens = a.seqlens;
  p.o = static_cast<char*>(a.o);
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
  p.block_table = a.block_table;
  p.page_size = a.page_size;
  p.pages_per_seq = a.pages_per_seq;
  p.num_pages = a.num_pages;
  p.Nq = a.Nq;
  p.ncg = (a.Nq * p.group + 15) / 16;
  p.causal = a.causal;
  p.n_new = a.k_new != nullptr ? a.Nq : 0;
  p.kn = static_cast<const char*>(a.k_new);
  p.vn = static_cast<const char*>(a.v_new);
  if (p.S > 1) {
    p.part_o = static_cast<float*>(a.workspace);
    p.part_lse = p.part_o + (size_t)a.B * a.Nq * a.Hq * p.S * D;
  }
  dim3 grid(a.Hkv * p.ncg, a.B, p.S);
  hipLaunchKernelGGL((decode_split_kernel<D, TL>), grid, dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  const int rows = a.B * a.Nq * a.Hq;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, stream, p, rows);
  return hipGetLastError();
}

// The balanced decode: at most 16 (query, query head) columns per pair, at
// least two parts per pair on average (num_splits - 1 units per pair).
template <int D, class TL>
hipError_t launch_lean(const DecodeArgs& a, hipStream_t stream, int64_t U) {
  DecParams p;
  p.q = static_cast<const char*>(a.q);
  p.kc = static_cast<char*>(const_cast<void*>(a.kcache));
  p.vc = static_cast<char*>(const_cast<void*>(a.vcache));
  p.lens = a.seqlens;
  p.o = static_cast<char*>(a.o);
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.capacity = a.capacity;
  p.S = a.num_splits;
  p.chunk = 0;
  p.c = a.scale * kLog2e;
  p.block_table = a.block_table;
  p.page_size = a.page_size;
  p.pages_per_seq = a.pages_per_seq;
  p.num_pages = a.num_pages;
  p.Nq = a.Nq;
  p.ncg = 1;
  p.causal = a.causal;
  p.n_new = a.k_new != nullptr ? a.Nq : 0;
  p.kn = static_cast<const char*>(a.k_new);
  p.vn = static_cast<const char*>(a.v_new);
  p.part_o = static_cast<float*>(a.workspace);
  p.part_lse = p.part_o + (size_t)a.B * a.Nq * a.Hq * p.S * D;
  const bool mq = a.Nq > 1 || a.k_new != nullptr;
  if (mq)
    hipLaunchKernelGGL((decode_lean_kernel<D, TL, true>), dim3((unsigned)U), dim3(64), 0, stream, p, a.B, U);
  else
    hipLaunchKernelGGL((decode_lean_kernel<D, TL, false>), dim3((unsigned)U), dim3(64), 0, stream, p, a.B, U);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = a.B * a.Nq * a.Hq;
  if (mq)
    hipLaunchKernelGGL((decode_lean_combine_kernel<D, TL::T, true>), dim3((rows + 3) / 4), dim3(256), 0, stream, p,
                       a.B, U);
  else
    hipLaunchKernelGGL((decode_lean_combine_kernel<D, TL::T, false>), dim3((rows + 3) / 4), dim3(256), 0, stream, p,
                       a.B, U);
  return hipGetLastError();
}

// Tile shape of the balanced decode per head dimension. At d = 64 and 128,
// calls with at least kLeanSmallTilePairs (sequence, key/value head) pairs
// take 32-key tiles (measured on MI355X, GQA with 8 KV heads: 2-4% faster
// from 32 sequences up at d = 128, 17% with short sequences, 1-2% at d = 64;
// 64-key tiles stay 6-11% faster at 8 sequences or fewer, whose defaults
// split each pair further).
template <int D>
using LeanTile = DecTile<D, (D <= 128 ? 64 : 32), 2>;
template <int D>
using LeanTileSmall = DecTile<D, 32, 2>;
constexpr int64_t kLeanSmallTilePairs = 256;
bool lean_small_tiles(int d, int64_t pairs) { return (d == 64 || d == 128) && pairs >= kLeanSmallTilePairs; }

// Units of the balanced decode, or 0 where it does not apply (no split, a
// shape decode_balanced turns away, or sizes whose unit arithmetic would
// leave 64-bit range).
int64_t lean_units(const DecodeArgs& a) {
  if (a.num_splits < 2 || !decode_balanced(a.B, a.Nq, a.Hq, a.Hkv, a.k_new != nullptr)) return 0;
  const int T = 32;  // the smallest tile any shape takes: the most tiles
  const int64_t U = (int64_t)(a.num_splits - 1) * a.B * a.Hkv;
  const double tiles = (double)a.B * a.Hkv * (((double)a.capacity + T - 1) / T);
  if (U > 0x7fffffff || tiles * (double)U >= 4.0e18) return 0;
  return U;
}

// Tile-shape override for tuning (FA_DEC_VARIANT), read once per process.
int dec_variant() {
  static const int v = [] {
    const char* e = getenv("FA_DEC_VARIANT");
    return e ? atoi(e) : 0;
  }();
  return v;
}

}  // namespace

// Whether a split decode call takes the balanced schedule: one query per
// sequence with nothing appended always; several queries or appended rows
// when their columns fit one MFMA group (Nq G <= 16) and there are at least
// 64 (sequence, key/value head) pairs. Below that the position splits were
// faster on MI355X (32 pairs, GQA 32/8, d = 128: 22.5 against 26.0 us),
// from 64 pairs on the balanced schedule (64 pairs: 64.2 against 70.3 us).
bool decode_balanced(int B, int Nq, int Hq, int Hkv, bool append) {
  if (B <= 0 || Hkv <= 0 || (int64_t)Nq * (Hq / Hkv) > 16) return false;
  return (Nq == 1 && !append) || (int64_t)B * Hkv >= 64;
}

int decode_chunk(int capacity, int num_splits) {
  const int per = (capacity + num_splits - 1) / num_splits;
  const int c = ((per + kSplitAlign - 1) / kSplitAlign) * kSplitAlign;
  return c > 0 ? c : kSplitAlign;
}

size_t decode_workspace_bytes(int B, int Hq, int d, int num_splits) {
  if (num_splits <= 1) return 0;
  return (size_t)B * Hq * num_splits * ((size_t)d + 1) * sizeof(float);
}

// Resident workgroups per CU of the balanced decode (its one-query form;
// the LDS ring and query buffers bound both forms alike).
int decode_resident_per_cu(int d, int64_t pairs) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (d) {
    case 64:
      e = lean_small_tiles(d, pairs)
              ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_lean_kernel<64, LeanTileSmall<64>, false>, 64, 0)
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_lean_kernel<64, LeanTile<64>, false>, 64, 0);
      break;
    case 128:
      e = lean_small_tiles(d, pairs)
              ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_lean_kernel<128, LeanTileSmall<128>, false>, 64, 0)
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_lean_kernel<128, LeanTile<128>, false>, 64, 0);
      break;
    case 256: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_lean_kernel<256, LeanTile<256>, false>, 64, 0); break;
    default: break;
  }
  if (e != hipSuccess) (void)hipGetLastError();  // leave no sticky error behind
  return e == hipSuccess && n > 0 ? n : 2;
}

int decode_split_resident_per_cu(int d) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (d) {
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_kernel<64, DecTile<64, 64, 3>>, 64, 0); break;
    case 128: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_kernel<128, DecTile<128, 64, 2>>, 64, 0); break;
    case 256: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_kernel<256, DecTile<256, 32, 2>>, 64, 0); break;
    default: break;
  }
  if (e != hipSuccess) (void)hipGetLastError();
  return e == hipSuccess && n > 0 ? n : 2;
}

bool decode_supported(int d, int group) {
  return (d == 64 || d == 128 || d == 256) && group >= 1 && group <= kMaxGroup;
}

// Tile shapes per head dimension, chosen by measurement on MI355X (d=128:
// 64-key tiles in a two-stage ring, two wavefronts per CU, beat 32-key
// tiles in three- or four-stage rings). FA_DEC_VARIANT selects the others.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (const int64_t U = lean_units(a)) {
    switch (a.d) {
      case 64:
        return lean_small_tiles(64, (int64_t)a.B * a.Hkv) ? launch_lean<64, LeanTileSmall<64>>(a, stream, U)
                                                         : launch_lean<64, LeanTile<64>>(a, stream, U);
      case 128:
        return lean_small_tiles(128, (int64_t)a.B * a.Hkv) ? launch_lean<128, LeanTileSmall<128>>(a, stream, U)
                                                          : launch_lean<128, LeanTile<128>>(a, stream, U);
      case 256: return launch_lean<256, LeanTile<256>>(a, stream, U);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.d) {
    case 64: return launch<64, DecTile<64, 64, 3>>(a, stream);
    case 128:
      switch (dec_variant()) {
        case 1: return launch<128, DecTile<128, 32, 4>>(a, stream);
        case 2: return launch<128, DecTile<128, 32, 2>>(a, stream);
        case 3: return launch<128, DecTile<128, 32, 3>>(a, stream);
        default: return launch<128, DecTile<128, 64, 2>>(a, stream);
      }
    case 256: return launch<256, DecTile<256, 32, 2>>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
