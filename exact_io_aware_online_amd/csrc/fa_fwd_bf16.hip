// fa_fwd_bf16.hip - prefill / training forward in bf16 for gfx950.
//
// One workgroup owns one tile of BM query rows of one (batch, query head)
// and streams every key/value tile those rows may see (FlashAttention:
// Part 2, section 1.2: query-row tiles are independent units of work;
// section 1.3: each wavefront owns whole rows, so no partial results cross
// wavefronts). Per key tile (FlashAttention: Part 2, section 6.2): score
// tile -> online softmax -> value accumulation -> discard; the N x N matrix
// never leaves registers.
//
// Data movement. K and V tiles go HBM -> LDS with direct-to-LDS 16-byte
// loads (global_load_lds_dwordx4) into an NST-stage ring, so a tile is in
// flight while earlier ones are consumed and no registers stage it. The
// loads are issued from inline assembly: the compiler does not track them,
// and the pipeline's own waits (vmcnt) and one s_barrier per tile order
// them. Inside a stage each row's 16-byte chunks are XOR-swizzled so the
// MFMA operand reads below hit distinct LDS banks.
//
// Math. The score tile is computed transposed, S^T = K Q^T, on the
// 32x32x16 bf16 MFMA: its accumulator gives each lane (lane % 32) a single
// query, so the running max, the running sum and the output column of that
// query live in that lane and the row max needs one exchange with the lane
// 32 away. P^T then feeds O^T += V^T P^T directly as the B operand. The
// V^T A operand is read from the row-major V tile with ds_read_b64_tr_b16,
// which transposes 16-bit elements across each group of 16 lanes.
//
// Softmax runs in base 2: t = s * scale * log2(e), the running maximum m in
// the same units, alpha = 2^(m - m') (FlashAttention: Part 2, section 6.2
// gives alpha = e^(m - m'); e^x = 2^(x log2 e)). The reference m is moved
// lazily: only when some row of the wavefront sees a score more than
// kSlack (8, base 2) above its current reference are m, l and the
// accumulator rescaled; otherwise probabilities 2^(t - m) stay below 2^8
// and both the accumulator and l keep the old reference, which leaves
// O = acc / l unchanged. Normalisation is deferred to the end
// (FlashAttention: Part 2, section 1.3), where the row's log-sum-exp is
// written as ln2 * (m + log2 l).
#include <type_traits>

#include <stdlib.h>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_fwd_tile_asm.h"

namespace fa {
namespace {

struct FwdParams {
  const char* __restrict__ q;
  const char* __restrict__ k;
  const char* __restrict__ v;
  char* __restrict__ o;
  float* __restrict__ lse;
  int Nq, Nk, Hq, Hkv, group, B;  // dense lengths (packed batches: Nq = longest sequence)
  // visible keys of query i: i + off - wl <= j <= i + off + wr (a negative
  // bound is unlimited), off = Nk_b - Nq_b when bottom_right, else 0;
  // top-left causal is (wl, wr) = (-1, 0)
  int wl, wr, bottom_right;
  int lpt;           // longest-first order (later query tiles see more keys)
  int hchunks;       // (sequence, key/value head) pairs run in this many consecutive chunks
  // packed variable-length batch: sequence b is rows cu_q[b] .. cu_q[b+1]
  // of q / o and cu_k[b] .. cu_k[b+1] of k / v; null for the dense layout
  const int32_t* __restrict__ cu_q;
  const int32_t* __restrict__ cu_k;
  int total_q, total_k;  // packed row counts (LSE is then (Hq, total_q))
  int n_qtiles;
  float c;  // scale * log2(e)
};

template <int D_, int BN_, int NW_, int QB_, int NST_, int WPS_, bool PIPE_ = false, bool ASM_ = false>
struct Cfg {
  static constexpr int D = D_, BN = BN_, NW = NW_, QB = QB_, NST = NST_;
  // one wavefront per SIMD, two query blocks per wavefront, each tile's
  // body one hand-scheduled statement (fa_fwd_tile_asm.h)
  static constexpr bool ASM = ASM_;
  static constexpr int WAVES_PER_SIMD = WPS_;  // register budget: 512 / WPS per lane
  // one wavefront per SIMD, two query blocks per wavefront, each tile's
  // MFMA phases overlapped with the other block's softmax (see the kernel)
  static constexpr bool PIPE = PIPE_;
  // ring stage as an immediate LDS offset (one copy of the tile code per
  // stage); head dimension 256 has no registers to spare for it
  static constexpr bool CONST_STAGE = D_ < 256;
  // issue priority raised for the S^T MFMA phase as well as the PV phase
  // (measured on MI355X: 4.4% faster at d = 256, 1.6% at d = 64; at d = 128
  // raising it for the PV phase alone is best)
  static constexpr bool PRIO_S = D_ != 128;
  // a computed tile requests the ring's next tile after its S^T MFMAs
  // rather than right after the barrier, so those loads land while the
  // softmax runs instead of beside the K operand reads (1.7% faster at
  // d = 256 on MI355X; no change at d = 64 and 128)
  static constexpr bool LATE_DMA = D_ == 256;
  static constexpr int BM = NW * 32 * QB;          // query rows per workgroup
  static constexpr int THREADS = NW * 64;
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * D * 2;    // one K (or V) tile
  // LDS ring: the NST K tiles, then the NST V tiles, so a read's stage
  // offset (stage * TILE_BYTES) plus its in-tile offset fits the 16-bit
  // immediate of an LDS instruction for every stage
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int V_REGION = NST_ * TILE_BYTES;
  static constexpr int DMA = TILE_BYTES / (THREADS * 16);  // 16-byte loads per thread per tile
  static_assert(DMA >= 1 && TILE_BYTES % (THREADS * 16) == 0, "tile does not split over the threads");
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shapes");
  static_assert(NST >= 2 && (NST - 2) * 2 * DMA <= 63, "vmcnt range");
};

// Growth of a row maximum (base-2 units) tolerated before the running
// maximum and the accumulator are rescaled.
constexpr float kSlack = 8.f;

template <class C>
__global__ __launch_bounds__(C::THREADS, C::WAVES_PER_SIMD) void fwd_bf16_kernel(FwdParams p) {
  constexpr int D = C::D, BN = C::BN, QB = C::QB, NST = C::NST, CPR = C::CPR;
  __shared__ __attribute__((aligned(1024))) char smem[NST * C::STAGE_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS3 char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches below
  const int g = lane >> 5;    // half of the wavefront
  const int r32 = lane & 31;  // query (S^T column) within a 32-row block

  // Work order (1-D grid). The (sequence, key/value head) pairs run in
  // hchunks consecutive chunks; within a chunk, rank r of the query tile is
  // outermost, so with a causal mask every head's longest tile is
  // dispatched before any shorter one (longest-processing-time order; the
  // short tiles fill the tail). Within a rank, workgroups that share a
  // key/value head sit a multiple of the chunk's pair count apart; with that
  // count a multiple of the 8 XCDs (dispatch goes round-robin over them)
  // they land on the same XCD and share its L2. Chunking halves the number
  // of heads whose K/V an XCD streams at once.
  const int pairs = p.Hkv * p.B / p.hchunks;  // pairs per chunk
  const int heads = pairs * p.group;           // workgroups per rank of a chunk
  const int hc = blockIdx.x / (heads * p.n_qtiles);
  const int bx = blockIdx.x - hc * heads * p.n_qtiles;
  const int r = bx / heads;
  const int rest = bx - r * heads;
  const int j = rest / pairs;
  const int pr = rest - j * pairs + hc * pairs;
  const int b = pr / p.Hkv;
  const int kvh = pr - b * p.Hkv;
  const int hq = kvh * p.group + j;
  const int qt = p.lpt ? p.n_qtiles - 1 - r : r;
  const int q0 = qt * C::BM;
  const int qw0 = q0 + wave * 32 * QB;  // first query row of this wavefront

  const int64_t q_row = (int64_t)p.Hq * D * 2;    // bytes between query rows
  const int kv_row = p.Hkv * D * 2;                // bytes between key rows

  // this sequence's rows (packed batches clamp the offsets into range)
  int qrow0, Nqb, krow0, Nkb;
  if (p.cu_q != nullptr) {
    qrow0 = min(max(p.cu_q[b], 0), p.total_q);
    const int lq = min(max(p.cu_q[b + 1], qrow0), p.total_q) - qrow0;
    krow0 = min(max(p.cu_k[b], 0), p.total_k);
    Nkb = min(max(p.cu_k[b + 1], krow0), p.total_k) - krow0;
    if (lq > p.Nq) {
      // longer than the grid's max_seqlen_q: every O and LSE row of the
      // sequence becomes NaN (the last query tile's workgroup also covers
      // the rows past the grid) rather than a partial result
      const int r1 = qt == p.n_qtiles - 1 ? lq : min(q0 + C::BM, lq);
      fill_nan_rows<D * 2>(p.o + (int64_t)qrow0 * p.Hq * D * 2 + (int64_t)hq * D * 2, (int64_t)p.Hq * D * 2, q0, r1,
                           tid, C::THREADS);
      if (p.lse != nullptr)
        for (int r = q0 + tid; r < r1; r += C::THREADS) p.lse[(int64_t)hq * p.total_q + qrow0 + r] = __builtin_nanf("");
      return;
    }
    Nqb = lq;
  } else {
    qrow0 = b * p.Nq;
    Nqb = p.Nq;
    krow0 = b * p.Nk;
    Nkb = p.Nk;
  }
  if (q0 >= Nqb) return;  // whole workgroup: past this sequence's queries
  const int off = p.bottom_right ? Nkb - Nqb : 0;
  // keys some row of the tile sees: tiles t0 .. t0 + ntiles - 1
  const int q_last = min(q0 + C::BM, Nqb) - 1;
  const int klo = p.wl >= 0 ? max(q0 + off - p.wl, 0) : 0;
  const int khi = p.wr >= 0 ? min(q_last + off + p.wr, Nkb - 1) : Nkb - 1;
  const int t0 = klo / BN;
  const int ntiles = khi >= klo ? khi / BN - t0 + 1 : 0;

  // ---- DMA addressing: load j of a tile fills slot j*THREADS + tid
  const char* kbase = p.k + ((int64_t)krow0 * p.Hkv + kvh) * D * 2;
  const char* vbase = p.v + ((int64_t)krow0 * p.Hkv + kvh) * D * 2;
  // load j of a tile fills slot s = j*THREADS + tid, i.e. row s / CPR; the
  // byte offsets of full tiles are computed once
  int dma_row[C::DMA], dma_col[C::DMA];
  uint32_t dma_off[C::DMA];
#pragma unroll
  for (int j = 0; j < C::DMA; ++j) {
    const int slot = j * C::THREADS + tid;
    dma_row[j] = slot / CPR;
    dma_col[j] = ((slot % CPR) ^ swz_pf<CPR>(slot / CPR)) * 16;
    dma_off[j] = (uint32_t)(dma_row[j] * kv_row + dma_col[j]);
  }
  const uint32_t dma_lds = __builtin_amdgcn_readfirstlane(lds0 + wave * 64 * 16);

  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    const int j0 = (t0 + t) * BN;
    const char* ks = kbase + (int64_t)j0 * kv_row;
    const char* vs = vbase + (int64_t)j0 * kv_row;
    const uint32_t st = dma_lds + (uint32_t)((t % NST) * C::TILE_BYTES);
    if (j0 + BN <= Nkb) {  // uniform: full tile
#pragma unroll
      for (int j = 0; j < C::DMA; ++j) dma16(ks, dma_off[j], st + j * C::THREADS * 16);
#pragma unroll
      for (int j = 0; j < C::DMA; ++j) dma16(vs, dma_off[j], st + C::V_REGION + j * C::THREADS * 16);
    } else {
      const int last = Nkb - 1 - j0;  // rows past the end re-read the last key (masked later)
#pragma unroll
      for (int j = 0; j < C::DMA; ++j)
        dma16(ks, (uint32_t)(min(dma_row[j], last) * kv_row + dma_col[j]), st + j * C::THREADS * 16);
#pragma unroll
      for (int j = 0; j < C::DMA; ++j)
        dma16(vs, (uint32_t)(min(dma_row[j], last) * kv_row + dma_col[j]), st + C::V_REGION + j * C::THREADS * 16);
    }
  };

  // ---- Q^T as B operand: register i of k-step ks = Q[row][16 ks + 8 g + i].
  // At d = 128, where the ring stage that is still free holds the tile's BM
  // query rows (BM <= 2 BN), they come in whole rows by direct-to-LDS
  // loads, requested before the first K/V tiles, and each wavefront reads
  // its operands from there (measured 2.3% faster on the short causal
  // workload, 0.6% slower at d = 64); otherwise every lane loads its
  // 16-byte pieces directly.
  constexpr bool STAGE_Q = D == 128 && C::BM <= 2 * BN;
  bf16x8 qf[QB][D / 16];
  if constexpr (STAGE_Q) {
    // rows [0, BN) of the tile into the K half of stage NST - 1, rows
    // [BN, 2 BN) into its V half; rows past the sequence re-read its last
    // query row (their operands are zeroed below)
    const char* qbase = p.q + ((int64_t)qrow0 + q0) * q_row + (int64_t)hq * D * 2;
    const int qlast = Nqb - 1 - q0;
#pragma unroll
    for (int h = 0; h < C::BM / BN; ++h) {
      const uint32_t st = dma_lds + (uint32_t)((h ? C::V_REGION : 0) + (NST - 1) * C::TILE_BYTES);
#pragma unroll
      for (int j = 0; j < C::DMA; ++j)
        dma16(qbase, (uint32_t)(min(h * BN + dma_row[j], qlast) * q_row + dma_col[j]), st + j * C::THREADS * 16);
    }
  }

  // start the K/V pipeline
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < ntiles) issue_tile(s);

  if constexpr (STAGE_Q) {
    // own Q loads landed when at most the K/V tiles issued after them remain
    const int issued = min(NST - 1, ntiles);
    static_for<NST>([&](auto A) {
      if (issued == decltype(A)::value) wait_vmcnt<decltype(A)::value * 2 * C::DMA>();
    });
    barrier();  // everyone's Q rows landed
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int trow = wave * 32 * QB + qb * 32 + r32;  // row within the tile
      const int lrow = trow % BN;
      const uint32_t base = lds0 + (uint32_t)((trow >= BN ? C::V_REGION : 0) + (NST - 1) * C::TILE_BYTES + lrow * D * 2);
      const int sw = swz_pf<CPR>(lrow);
      const bool valid = qw0 + qb * 32 + r32 < Nqb;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 x = *(const LDS3 bf16x8*)(uintptr_t)(base + (((2 * ks + g) ^ sw) * 16));
        qf[qb][ks] = valid ? x : bf16x8{};
      }
    }
    // the reads complete before the barrier after which tile NST - 1 refills this stage
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited on
  } else {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = qw0 + qb * 32 + r32;
      const char* qrow = p.q + ((int64_t)qrow0 + row) * q_row + (int64_t)hq * D * 2;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        qf[qb][ks] = row < Nqb ? *reinterpret_cast<const bf16x8*>(qrow + (ks * 16 + g * 8) * 2) : bf16x8{};
      }
    }
    wait_vm_loads();
  }

  f32x16 acc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[qb][dt] = f32x16{};
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;  // running max of t, base-2 units
    l[qb] = 0.f;        // running sum of 2^(t - m) over this lane's keys
  }

  // ---- per-lane LDS read offsets within a stage (the parts that vary by
  // 32-key block nb or 16-key block kk are compile-time immediates). With
  // 16 or more chunks per row the swizzle is below 16 and only permutes a
  // chunk index's low four bits, so k-steps ks and ks + 8, and 32-column
  // blocks dt and dt + 4, sit exactly 256 bytes apart: one register per
  // residue, the rest an immediate (16 registers fewer at d = 256).
  constexpr int NKO = (CPR >= 16 && D / 16 > 8) ? 8 : D / 16;
  constexpr int NVO = (CPR >= 16 && D / 32 > 4) ? 4 : D / 32;
  // K (b128): row = 32 nb + r32, logical chunk 2 ks + g
  uint32_t k_off[NKO];
  {
    const int ksw = swz_pf<CPR>(r32);
#pragma unroll
    for (int ks = 0; ks < NKO; ++ks) k_off[ks] = (uint32_t)(r32 * D * 2 + (((2 * ks + g) ^ ksw) * 16));
  }
  auto kofs = [&](int ks) __attribute__((always_inline)) { return k_off[ks % NKO] + (uint32_t)(ks / NKO) * 256u; };
  // V (transposed b64): 16-lane group grp = lane / 16 reads rows
  // 16 kk + 8 h + 4 g + (lane % 16) / 4 at columns 32 dt + 16 (grp % 2) + 4 (lane % 4)
  uint32_t v_off[NVO][2];
  {
    const int vi = lane & 15;
    const int vgrp = lane >> 4;
    const int vcol = (vgrp & 1) * 2 + ((vi & 3) >> 1);  // logical chunk within a 32-column block
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * h + 4 * (vgrp >> 1) + (vi >> 2);
      const int sw = swz_pf<CPR>(row);
#pragma unroll
      for (int dt = 0; dt < NVO; ++dt)
        v_off[dt][h] = (uint32_t)(C::V_REGION + row * D * 2 + (vi & 1) * 8 + (((4 * dt + vcol) ^ sw) * 16));
    }
  }
  auto vofs = [&](int dt, int h) __attribute__((always_inline)) {
    return v_off[dt % NVO][h] + (uint32_t)(dt / NVO) * 256u;
  };

  // Every wavefront takes part in every tile's wait + barrier + prefetch,
  // in order; it computes on tiles [0, nt_w), of which the first nt_full
  // need no mask. Peeling the loop this way keeps the accumulator's
  // loop-carried registers free of branches.
  auto sync_wait = [&](int t) __attribute__((always_inline)) {
    // own loads of tile t are done when at most those of the tiles issued
    // after it (t+1 .. t+NST-2, within range) remain
    const int after = min(NST - 2, ntiles - 1 - t);
    static_for<NST - 1>([&](auto A) {
      if (after == decltype(A)::value) wait_vmcnt<decltype(A)::value * 2 * C::DMA>();
    });
    barrier();  // everyone's loads of tile t landed; tile t-1 is no longer read
  };
  auto sync_tile = [&](int t) __attribute__((always_inline)) {
    sync_wait(t);
    if (t + NST - 1 < ntiles) issue_tile(t + NST - 1);
  };
  // before a tile this wavefront computes (with LATE_DMA the tile itself
  // requests its successor, after its S^T phase)
  auto sync_compute = [&](int t) __attribute__((always_inline)) {
    if constexpr (C::LATE_DMA) sync_wait(t);
    else sync_tile(t);
  };

  constexpr int NBT = BN / 32;
  f32x16 sc[QB][NBT];     // scores of a tile, from its S phase to its softmax
  bf16x8 pf[QB][BN / 16]; // its P^T, from the softmax to its PV phase

  // S^T = K Q^T for tile t held in ring stage `stage` (given as a
  // compile-time constant, every LDS read address is a per-lane register
  // plus an immediate): BN keys x 32 queries per query block. The K
  // operands are read KPF ahead of their MFMA so LDS latency overlaps the
  // chain (at d = 128 all of them first: 1-2% faster on the long causal
  // workload than eight ahead).
  auto s_phase = [&](int t, auto stage) __attribute__((always_inline)) {
    const uint32_t stg = (uint32_t)(int)stage * C::TILE_BYTES;
    constexpr int NK = (D / 16) * NBT;
    constexpr int KPF = D >= 256 ? 2 : (D == 128 ? NK : (NK < 8 ? NK : 8));
    auto kread = [&](int i) __attribute__((always_inline)) {
      return *(const LDS3 bf16x8*)(uintptr_t)(lds0 + stg + kofs(i / NBT) + (i % NBT) * 32 * D * 2);
    };
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb) sc[qb][nb] = f32x16{};
    bf16x8 kf[NK];
#pragma unroll
    for (int i = 0; i < KPF; ++i) kf[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the chain
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      if (i + KPF < NK) kf[i + KPF] = kread(i + KPF);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb][i % NBT] = mfma32x32x16(kf[i], qf[qb][i / NBT], sc[qb][i % NBT]);
    }
  };

  // online softmax of tile t: mask, running max, lazy rescale of l and the
  // accumulator, probabilities and their row sums, P^T packed to bf16
  auto softmax_phase = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int j0 = (t0 + t) * BN;
    bool moved = false;
    float alpha[QB], m_cand[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if constexpr (MASK) {
        // key j0 + 4g + o (o = 32 nb + 8 (i/4) + i%4) is visible iff lo <= o <= hi
        const int my_q = qw0 + qb * 32 + r32;
        const int base = j0 + 4 * g;
        const int lo = (p.wl >= 0 ? my_q + off - p.wl : 0) - base;
        const int hi = (p.wr >= 0 ? min(my_q + off + p.wr, Nkb - 1) : Nkb - 1) - base;
#pragma unroll
        for (int nb = 0; nb < NBT; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int o = nb * 32 + 8 * (i >> 2) + (i & 3);
            if (o < lo || o > hi) sc[qb][nb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[qb][nb][i]);
      mx = halves_max(mx);
      m_cand[qb] = fmaxf(m[qb], mx * p.c);
      moved |= m_cand[qb] > m[qb] + kSlack;
    }
    // The running max only moves when some row's max grew by more than
    // kSlack: below that, probabilities 2^(t - m) stay <= 2^kSlack, exact
    // in fp32/bf16 range, and O = acc / l is unchanged because acc and l
    // share the same reference m.
    const bool rescale = __builtin_amdgcn_ballot_w64(moved) != 0;  // wave-uniform
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (rescale) {
        const float mu = (m_cand[qb] == -INFINITY) ? 0.f : m_cand[qb];  // never (-inf) - (-inf)
        alpha[qb] = exp2_fast(m[qb] - mu);
        l[qb] *= alpha[qb];
        m[qb] = m_cand[qb];
      }
      const float m_use = (m[qb] == -INFINITY) ? 0.f : m[qb];
      // row sum as a pairwise tree: a short dependency chain
      float e[NBT * 16];
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = exp2_fast(fmaf(sc[qb][nb][i], p.c, -m_use));
          sc[qb][nb][i] = pv;
          e[nb * 16 + i] = pv;
        }
#pragma unroll
      for (int w = NBT * 16 / 2; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) e[i] += e[i + w];
      l[qb] += e[0];
    }

    // P^T as B operands: 16-key step kk takes registers 8 (kk % 2) .. +7 of
    // accumulator kk / 2 (keys 8 (i / 4) + 4 g + i % 4 of that half).
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kk = 0; kk < BN / 16; ++kk) {
        const int nb = kk >> 1, h = (kk & 1) * 8;
        u32x4 w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) w[e2] = pack_bf16x2(sc[qb][nb][h + 2 * e2], sc[qb][nb][h + 2 * e2 + 1]);
        pf[qb][kk] = __builtin_bit_cast(bf16x8, w);
      }

    if (rescale) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[qb][dt] *= alpha[qb];
    }
  };

  // O^T += V^T P^T for tile t held in ring stage `stage`. Where registers
  // allow (one query block, d <= 128), the V^T operands of the next
  // 32-column block are read while the current block's MFMAs run (two
  // register sets), so each MFMA waits on reads issued a block earlier
  // rather than just before it.
  auto pv_phase = [&](int t, auto stage) __attribute__((always_inline)) {
    const uint32_t stg = (uint32_t)(int)stage * C::TILE_BYTES;
    constexpr int NKK = BN / 16, NDT = D / 32;
    constexpr bool AHEAD = QB == 1 && D <= 128;
    i16x4 vr[AHEAD ? 2 : 1][NKK][2];
    auto rd = [&](int dt, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h) vr[buf][kk][h] = ds_read_tr(lds0 + stg + vofs(dt, h) + kk * 16 * D * 2);
    };
    if constexpr (AHEAD) rd(0, 0);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int buf = AHEAD ? dt & 1 : 0;
      if constexpr (AHEAD) {
        if (dt + 1 < NDT) rd(dt + 1, (dt + 1) & 1);
      } else {
        rd(dt, 0);
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        // registers 0..3: keys 4 g + r; 4..7: keys 8 + 4 g + r (of block kk)
        const i16x4 v0 = vr[buf][kk][0], v1 = vr[buf][kk][1];
        const i16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        const bf16x8 va = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][dt] = mfma32x32x16(va, pf[qb][kk], acc[qb][dt]);
      }
    }
    if constexpr (AHEAD) {
      // issue order: the first block's reads, then each MFMA preceded by
      // two reads of the next block
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NKK, 0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          if (dt + 1 < NDT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    }
  };

  // the whole tile in one wavefront: S, softmax, then the PV block at
  // raised issue priority (and the S block too where PRIO_S): with two
  // wavefronts per SIMD, one then streams its MFMAs while the other works
  // through its softmax on the vector ALU.
  auto compute_tile = [&](int t, auto mask_tag, auto stage) __attribute__((always_inline)) {
    if constexpr (C::PRIO_S) {
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
    }
    s_phase(t, stage);
    if constexpr (C::PRIO_S) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (C::LATE_DMA) {
      __builtin_amdgcn_sched_barrier(0);
      if (t + NST - 1 < ntiles) issue_tile(t + NST - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    softmax_phase(t, mask_tag);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    pv_phase(t, stage);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };

  // tile t in its ring stage t % NST (uniform), for loops whose trip count
  // is not a multiple of NST
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

  // This wavefront's tiles (relative to t0): [t_lo, t_hi) hold a key some
  // of its rows see, [u_lo, u_hi) only keys all of its rows see (no mask).
  int t_lo = 0, t_hi = 0, u_lo = 0, u_hi = 0;
  {
    const int wq_last = min(qw0 + 32 * QB, Nqb) - 1;
    const int wlo = p.wl >= 0 ? max(qw0 + off - p.wl, 0) : 0;
    const int whi = p.wr >= 0 ? min(wq_last + off + p.wr, Nkb - 1) : Nkb - 1;
    if (wq_last >= qw0 && whi >= wlo) {
      t_lo = max(wlo / BN - t0, 0);
      t_hi = min(whi / BN - t0 + 1, ntiles);
      const int flo = p.wl >= 0 ? max(wq_last + off - p.wl, 0) : 0;
      const int fhi = p.wr >= 0 ? min(qw0 + off + p.wr, Nkb - 1) : Nkb - 1;
      u_lo = min(max((flo + BN - 1) / BN - t0, t_lo), t_hi);
      u_hi = min(max((fhi + 1) / BN - t0, u_lo), t_hi);
    }
  }
  if constexpr (C::ASM) {
    // The hand-scheduled 64-row shape. Fixed registers between the
    // statements below: O^T in a[0:127], the Q^T operands in a[128:191], the
    // V^T operands in a[192:255], the next tile's K operands in v[192:255];
    // LDS and DMA addresses enter in v[40:63]. Loads, waits and barriers of
    // tiles this wavefront does not compute, and loads of partial tiles,
    // stay here; each computed tile's statement waits for the next tile,
    // passes the barrier and issues the next-but-one tile's loads itself
    // (flags), so the next tile's K operands are read under its last MFMAs.
    static_assert(D == 128 && BN == 64 && QB == 2 && NST == 2 && C::NW == 2 && C::DMA == 8, "assembly tile shape");
    typedef uint32_t u32x32 __attribute__((ext_vector_type(32)));
    typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
    typedef float f32x32 __attribute__((ext_vector_type(32)));
    {
      u32x32 q0, q1;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 a = __builtin_bit_cast(u32x4, qf[0][ks]), b = __builtin_bit_cast(u32x4, qf[1][ks]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          q0[4 * ks + e] = a[e];
          q1[4 * ks + e] = b[e];
        }
      }
      asm volatile(FA_Q_TO_AGPR_ASM :: "{v[72:103]}"(q0), "{v[104:135]}"(q1) : FA_AGPR_CLOBBERS);
      asm volatile(FA_O_ZERO_ASM ::: FA_AGPR_CLOBBERS);
    }
    u32x8 kaddr, vaddr, doff;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kaddr[ks] = lds0 + kofs(ks);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h) vaddr[2 * dt + h] = lds0 + vofs(dt, h);
#pragma unroll
    for (int j = 0; j < 8; ++j) doff[j] = dma_off[j];
    float mA = m[0], mB = m[1], lA = l[0], lB = l[1];
    const uint32_t dl = dma_lds;
    // visible keys of block qb's row in tile t as lo .. lo + range relative
    // to key (t0 + t) BN + 4 g (an empty set as lo = 2^20, range = 0)
    auto mask_of = [&](int t, int qb, int& lo, int& range) __attribute__((always_inline)) {
      const int my_q = qw0 + qb * 32 + r32;
      const int base = (t0 + t) * BN + 4 * g;
      const int l0 = (p.wl >= 0 ? my_q + off - p.wl : 0) - base;
      const int h0 = (p.wr >= 0 ? min(my_q + off + p.wr, Nkb - 1) : Nkb - 1) - base;
      lo = h0 >= l0 ? l0 : (1 << 20);
      range = h0 >= l0 ? h0 - l0 : 0;
    };
    auto full_tile = [&](int t) __attribute__((always_inline)) { return (t0 + t + 1) * BN <= Nkb; };
    sync_tile(0);
    for (int t = 0; t < ntiles; ++t) {
      if (t < t_lo || t >= t_hi) {
        if (t + 1 < ntiles) sync_tile(t + 1);
        continue;
      }
      const int stage = t & 1;
      if (t == t_lo) {
        if (stage == 0)
          asm volatile(FA_KREAD_ASM_S0 :: "{v[40:47]}"(kaddr) : FA_KREAD_ASM_CLOBBERS);
        else
          asm volatile(FA_KREAD_ASM_S1 :: "{v[40:47]}"(kaddr) : FA_KREAD_ASM_CLOBBERS);
      }
      const bool dma_here = t + 2 < ntiles && full_tile(t + 2);
      const uint32_t fl = __builtin_amdgcn_readfirstlane((t + 1 < ntiles ? 1u : 0u) | (dma_here ? 2u : 0u) |
                                                         (t + 1 < t_hi ? 4u : 0u));
      const int64_t nxt = (int64_t)(t0 + t + 2) * BN * kv_row;
      const char* kb = kbase + (dma_here ? nxt : 0);
      const char* vb = vbase + (dma_here ? nxt : 0);
      const uint64_t kbu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)kb) |
                           ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uintptr_t)kb >> 32)) << 32);
      const uint64_t vbu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)vb) |
                           ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uintptr_t)vb >> 32)) << 32);
      const bool masked = t < u_lo || t >= u_hi;
      int loA = 0, rgA = 0, loB = 0, rgB = 0;
      if (masked) {
        mask_of(t, 0, loA, rgA);
        mask_of(t, 1, loB, rgB);
      }
      uint64_t sp;
#define FA_TILE_OPERANDS                                                                                      \
  : [mA] "+v"(mA), [mB] "+v"(mB), [lA] "+v"(lA), [lB] "+v"(lB), [sp] "=&s"(sp)                                \
  : [c] "s"(p.c), [fl] "s"(fl), [dl] "s"(dl), [kb] "s"(kbu), [vb] "s"(vbu), [loA] "v"(loA), [rgA] "v"(rgA), \
    [loB] "v"(loB), [rgB] "v"(rgB), "{v[40:47]}"(kaddr), "{v[48:55]}"(vaddr), "{v[56:63]}"(doff)            \
  : FA_TILE_ASM_CLOBBERS
      if (masked) {
        if (stage == 0)
          asm volatile(FA_TILE_ASM_S0_M FA_TILE_OPERANDS);
        else
          asm volatile(FA_TILE_ASM_S1_M FA_TILE_OPERANDS);
      } else {
        if (stage == 0)
          asm volatile(FA_TILE_ASM_S0_U FA_TILE_OPERANDS);
        else
          asm volatile(FA_TILE_ASM_S1_U FA_TILE_OPERANDS);
      }
#undef FA_TILE_OPERANDS
      (void)sp;
      // a partial next-but-one tile: its clamped loads from here, after the
      // statement's barrier
      if (t + 2 < ntiles && !dma_here) issue_tile(t + 2);
    }
    {
      f32x32 o0, o1, o2, o3;
      asm volatile(FA_O_READ_ASM : "={v[72:103]}"(o0), "={v[104:135]}"(o1), "={v[136:167]}"(o2), "={v[168:199]}"(o3)
                   :: FA_AGPR_CLOBBERS);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[0][0][i] = o0[i];
        acc[0][1][i] = o0[16 + i];
        acc[0][2][i] = o1[i];
        acc[0][3][i] = o1[16 + i];
        acc[1][0][i] = o2[i];
        acc[1][1][i] = o2[16 + i];
        acc[1][2][i] = o3[i];
        acc[1][3][i] = o3[16 + i];
      }
    }
    m[0] = mA;
    m[1] = mB;
    l[0] = lA;
    l[1] = lB;
  } else if constexpr (C::PIPE) {
    // Software pipeline of one wavefront per SIMD over two 32-row query
    // blocks A and B (64 rows), 32-key tiles. Every K and V^T operand is
    // read from LDS once per tile, held in registers, and feeds two MFMAs,
    // one per block: half the LDS bytes per flop of the one-block shape.
    // With no second wavefront on the SIMD to fill the matrix pipe during a
    // softmax, the wavefront overlaps its own, skewed by half a tile so
    // that every MFMA phase has softmax work beside it:
    //   P1: S_A(t) = K Q_A^T        | softmax(B, t-1) second half
    //   P2: O_B += V^T P_B^T (t-1)  | softmax(A, t) first half
    //   P3: S_B(t) = K Q_B^T        | softmax(A, t) second half; V^T(t) operands read
    //   (wait + barrier for tile t+1, its loads issued)
    //   P4: O_A += V^T P_A^T (t)    | softmax(B, t) first half; K(t+1) operands read
    // (FlashAttention: Part 2, section 1.5: overlap the softmax of one part
    // of the work with the matrix products of another.) Inside a phase each
    // MFMA is followed by one step of the softmax, with scheduling fences
    // between them, so the issue order is exactly that: the matrix pipe
    // runs the MFMA while the vector ALU runs the step.
    static_assert(QB == 2 && BN == 32 && NBT == 1, "pipelined shape");
    constexpr int NK = D / 16;           // K operands (and S MFMAs) per tile and block
    constexpr int NDT = D / 32;          // V^T blocks: PV MFMAs per tile and block = 2 NDT
    static_assert(NK == 8 && NDT == 4, "the step schedule below assumes d = 128");
    bf16x8 kf[NK];
    i16x4 vr[NDT][2][2];
    float mu[2];       // reference of the block's probabilities of its current tile
    float alpha[2];    // its rescale factor, applied to the accumulator before its PV
    bool rs[2];        // whether the reference moved (wave-uniform)
    float mx[2];

    auto fence = [] __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
    auto stage_of = [&](int t) __attribute__((always_inline)) {
      return (uint32_t)__builtin_amdgcn_readfirstlane((t % NST) * C::TILE_BYTES);
    };
    auto kread = [&](uint32_t stg, int i) __attribute__((always_inline)) {
      kf[i] = *(const LDS3 bf16x8*)(uintptr_t)(lds0 + stg + kofs(i));
    };
    auto vread = [&](uint32_t stg, int i) __attribute__((always_inline)) {  // i = 0 .. 15
      const int dt = i >> 2, kk = (i >> 1) & 1, h = i & 1;
      vr[dt][kk][h] = ds_read_tr(lds0 + stg + vofs(dt, h) + kk * 16 * D * 2);
    };
    auto mfma_s = [&](int qb, int i) __attribute__((always_inline)) {
      sc[qb][0] = mfma32x32x16(kf[i], qf[qb][i], i == 0 ? f32x16{} : sc[qb][0]);
    };
    auto mfma_pv = [&](int qb, int i) __attribute__((always_inline)) {
      const int dt = i >> 1, kk = i & 1;
      const i16x4 v0 = vr[dt][kk][0], v1 = vr[dt][kk][1];
      const i16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      acc[qb][dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, vv), pf[qb][kk], acc[qb][dt]);
    };
    auto expv = [&](int qb, int i) __attribute__((always_inline)) {
      sc[qb][0][i] = exp2_fast(fmaf(sc[qb][0][i], p.c, -mu[qb]));
      materialize(sc[qb][0][i]);
    };
    // First half of block qb's online softmax of tile t, in 8 steps: mask,
    // row maximum, the (lazy, as in the one-block shape) reference move,
    // and the first 10 of the 16 probabilities of this lane.
    auto sm1 = [&](int s, int t, int qb, auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      if (s <= 1) {
        if constexpr (MASK) {
          const int my_q = qw0 + qb * 32 + r32;
          const int base = (t0 + t) * BN + 4 * g;
          const int lo = (p.wl >= 0 ? my_q + off - p.wl : 0) - base;
          const int hi = (p.wr >= 0 ? min(my_q + off + p.wr, Nkb - 1) : Nkb - 1) - base;
#pragma unroll
          for (int i = 8 * s; i < 8 * s + 8; ++i) {
            const int o = 8 * (i >> 2) + (i & 3);
            if (o < lo || o > hi) sc[qb][0][i] = -INFINITY;
          }
        }
        float x = s == 0 ? fmaxf(sc[qb][0][0], sc[qb][0][1]) : fmaxf(mx[qb], fmaxf(sc[qb][0][8], sc[qb][0][9]));
#pragma unroll
        for (int i = 8 * s + 2; i < 8 * s + 8; ++i) x = fmaxf(x, sc[qb][0][i]);
        mx[qb] = x;
        materialize(x);
      } else if (s == 2) {
        const float m_cand = fmaxf(m[qb], halves_max(mx[qb]) * p.c);
        rs[qb] = __builtin_amdgcn_ballot_w64(m_cand > m[qb] + kSlack) != 0;  // wave-uniform
        const float m_new = rs[qb] ? m_cand : m[qb];
        mu[qb] = (m_new == -INFINITY) ? 0.f : m_new;  // never (-inf) - (-inf)
        alpha[qb] = rs[qb] ? exp2_fast(m[qb] - mu[qb]) : 1.f;
        m[qb] = m_new;
        materialize(mu[qb]);
        materialize(alpha[qb]);
      } else if (s == 3) {
        l[qb] *= alpha[qb];
        expv(qb, 0);
        expv(qb, 1);
        materialize(l[qb]);
      } else {
        expv(qb, 2 * s - 6);  // s = 4 .. 7: probabilities 2 .. 9
        expv(qb, 2 * s - 5);
      }
    };
    // Second half, in 8 steps: the last 6 probabilities, P^T packed to
    // bf16, and the row sum (after the packing, in place).
    auto sm2 = [&](int s, int qb) __attribute__((always_inline)) {
      if (s <= 2) {
        expv(qb, 10 + 2 * s);
        expv(qb, 11 + 2 * s);
      } else if (s <= 4) {
        const int kk = s - 3;
        u32x4 w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) w[e2] = pack_bf16x2(sc[qb][0][8 * kk + 2 * e2], sc[qb][0][8 * kk + 2 * e2 + 1]);
        pf[qb][kk] = __builtin_bit_cast(bf16x8, w);
        materialize(pf[qb][kk]);
      } else if (s == 5) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          sc[qb][0][i] += sc[qb][0][i + 8];
          materialize(sc[qb][0][i]);
        }
      } else if (s == 6) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[qb][0][i] += sc[qb][0][i + 4];
        sc[qb][0][0] += sc[qb][0][2];
        sc[qb][0][1] += sc[qb][0][3];
        materialize(sc[qb][0][0]);
        materialize(sc[qb][0][1]);
      } else {
        l[qb] += sc[qb][0][0] + sc[qb][0][1];
        materialize(l[qb]);
      }
    };
    auto rescale_acc = [&](int qb) __attribute__((always_inline)) {
      if (rs[qb]) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) scale_agpr16(acc[qb][dt], alpha[qb]);
      }
    };

    // one tile of this wavefront (kf holds K(t); block B's softmax of the
    // previous tile is half done and its PV pending)
    auto tile = [&](int t, auto mask_tag) __attribute__((always_inline)) {
      const uint32_t stg = stage_of(t);
      // P1
      static_for<8>([&](auto I) {
        mfma_s(0, I);
        fence();
        sm2(I, 1);
        fence();
      });
      rescale_acc(1);
      fence();
      // P2
      static_for<8>([&](auto I) {
        mfma_pv(1, I);
        fence();
        sm1(I, t, 0, mask_tag);
        fence();
      });
      // P3
      static_for<8>([&](auto I) {
        mfma_s(1, I);
        fence();
        sm2(I, 0);
        vread(stg, 2 * I);
        vread(stg, 2 * I + 1);
        fence();
      });
      rescale_acc(0);
      // tile t + 1 landed; the stage of tile t - 1 is refilled
      if (t + 1 < ntiles) sync_tile(t + 1);
      fence();
      // P4
      const uint32_t nstg = stage_of(t + 1);
      static_for<8>([&](auto I) {
        mfma_pv(0, I);
        fence();
        sm1(I, t, 1, mask_tag);
        kread(nstg, I);
        fence();
      });
    };
    // a tile this wavefront does not compute: keep the workgroup's order
    auto idle = [&](int t) __attribute__((always_inline)) {
      if (t + 1 < ntiles) sync_tile(t + 1);
      const uint32_t nstg = stage_of(t + 1);
#pragma unroll
      for (int i = 0; i < NK; ++i) kread(nstg, i);
    };

    // Block B starts with a pending tile that contributes nothing: zero
    // probabilities (the first half already "exponentiated" to 0, the rest
    // at -inf) and zero V^T operands.
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[1][0][i] = i < 10 ? 0.f : -INFINITY;
    mu[1] = 0.f;
    alpha[1] = 1.f;
    rs[1] = false;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) vr[dt][kk][0] = vr[dt][kk][1] = i16x4{};

    // the tiles in order, peeled into runs of one kind (one loop each keeps
    // the register allocation of every loop free of merged copies)
    sync_tile(0);
    {
      const uint32_t stg0 = stage_of(0);
#pragma unroll
      for (int i = 0; i < NK; ++i) kread(stg0, i);
    }
    int t = 0;
    for (; t < t_lo; ++t) idle(t);
    for (; t < u_lo; ++t) tile(t, std::true_type{});
    for (; t < u_hi; ++t) tile(t, std::false_type{});
    for (; t < t_hi; ++t) tile(t, std::true_type{});
    // drain: block B's last tile
    static_for<8>([&](auto I) { sm2(I, 1); });
    rescale_acc(1);
    static_for<8>([&](auto I) { mfma_pv(1, I); });
    for (; t < ntiles; ++t) idle(t);
  } else {
  int t = 0;
  for (; t < t_lo; ++t) sync_tile(t);
  for (; t < u_lo; ++t) {
    sync_compute(t);
    compute_any(t, std::true_type{});
  }
  if constexpr (C::CONST_STAGE) {
    for (; t < u_hi && t % NST != 0; ++t) {
      sync_compute(t);
      compute_any(t, std::false_type{});
    }
    // unmasked tiles NST at a time: tile t + S sits in stage S
    for (; t + NST <= u_hi; t += NST) {
      static_for<NST>([&](auto S) {
        sync_compute(t + decltype(S)::value);
        compute_tile(t + decltype(S)::value, std::false_type{}, S);
      });
    }
  }
  for (; t < u_hi; ++t) {
    sync_compute(t);
    compute_any(t, std::false_type{});
  }
  for (; t < t_hi; ++t) {
    sync_compute(t);
    compute_any(t, std::true_type{});
  }
  for (; t < ntiles; ++t) sync_tile(t);
  }

  // ---- epilogue: combine the two lane halves' sums, normalise once. At
  // d = 64 and 128 (where the ring has room) the normalised rows go through
  // LDS, idle now, so that each store writes whole rows: 16 lanes x 16
  // bytes per row at d = 128, instead of 8-byte pieces of 32 rows per
  // instruction. Those stores are non-temporal: O is written once and never
  // read here, so its lines go to memory now rather than sitting dirty in
  // the caches until a later kernel's traffic evicts them. At d = 256
  // staging costs registers the kernel does not have; there the rows are
  // stored from the accumulators as ordinary stores (partial lines written
  // past the caches are slow).
  constexpr int ROWB = D * 2;        // bytes of one O row
  constexpr int WROWS = 32 * QB;     // rows of this wavefront
  constexpr bool STAGE_O = D <= 128 && C::NW * WROWS * ROWB <= NST * C::STAGE_BYTES;
  if constexpr (STAGE_O) {
    const uint32_t ost = lds0 + (uint32_t)(wave * WROWS * ROWB);
    // 16-byte chunk c of row r sits at chunk c ^ (r % CPR), which spreads
    // the writes below (one chunk of 32 rows per instruction) over the banks
    barrier();  // every wavefront is done reading the ring
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = qb * 32 + r32;
      const int my_q = qw0 + row;
      const float lt = halves_sum(l[qb]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = dt * 4 + j;  // chunk of dims 8c .. 8c+7; this lane's half g holds 8c + 4g ..
          u32x2 w;
          w[0] = pack_bf16x2(acc[qb][dt][4 * j + 0] * inv, acc[qb][dt][4 * j + 1] * inv);
          w[1] = pack_bf16x2(acc[qb][dt][4 * j + 2] * inv, acc[qb][dt][4 * j + 3] * inv);
          *(LDS3 u32x2*)(uintptr_t)(ost + row * ROWB + ((c ^ (row % CPR)) * 16) + g * 8) = w;
        }
      }
      if (p.lse != nullptr && g == 0 && my_q < Nqb) {
        const int64_t lrow = p.cu_q != nullptr ? (int64_t)hq * p.total_q + qrow0 : ((int64_t)b * p.Hq + hq) * p.Nq;
        p.lse[lrow + my_q] = lt > 0.f ? (m[qb] + log2_fast(lt)) * kLn2 : -INFINITY;
      }
    }
    // each wavefront reads back only its own rows: no barrier, the LDS
    // instructions of one wavefront complete in order
#pragma unroll
    for (int i = 0; i < WROWS * CPR / 64; ++i) {
      const int slot = i * 64 + lane;
      const int row = slot / CPR, c = slot % CPR;
      const u32x4 w = *(const LDS3 u32x4*)(uintptr_t)(ost + row * ROWB + ((c ^ (row % CPR)) * 16));
      const int my_q = qw0 + row;
      if (my_q < Nqb)
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p.o + ((int64_t)qrow0 + my_q) * q_row +
                                                                (int64_t)hq * D * 2 + c * 16));
    }
  } else {
    // stores straight from the accumulators (this code shape keeps the
    // d = 256 kernel's register allocation at its measured best)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int my_q = qw0 + qb * 32 + r32;
      const float lt = halves_sum(l[qb]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      if (my_q < Nqb) {
        char* orow = p.o + ((int64_t)qrow0 + my_q) * q_row + (int64_t)hq * D * 2;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d0 = dt * 32 + 8 * j + 4 * g;
            u32x2 w;
            w[0] = pack_bf16x2(acc[qb][dt][4 * j + 0] * inv, acc[qb][dt][4 * j + 1] * inv);
            w[1] = pack_bf16x2(acc[qb][dt][4 * j + 2] * inv, acc[qb][dt][4 * j + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + d0 * 2) = w;
          }
        }
        if (p.lse != nullptr && g == 0) {
          const int64_t lrow = p.cu_q != nullptr ? (int64_t)hq * p.total_q + qrow0 : ((int64_t)b * p.Hq + hq) * p.Nq;
          p.lse[lrow + my_q] =
              lt > 0.f ? (m[qb] + log2_fast(lt)) * kLn2 : -INFINITY;
        }
      }
    }
  }
}

template <class C>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  p.q = static_cast<const char*>(a.q);
  p.k = static_cast<const char*>(a.k);
  p.v = static_cast<const char*>(a.v);
  p.o = static_cast<char*>(a.o);
  p.lse = a.lse;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.wl = a.window_left;
  p.wr = a.window_right;
  p.bottom_right = a.bottom_right;
  p.lpt = a.window_right >= 0;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  p.n_qtiles = (a.Nq + C::BM - 1) / C::BM;
  // two chunks where each still spreads over all 8 XCDs (measured 2.4% faster
  // on the causal B8 H16 N2048 workload: more of the streamed K/V hits L2)
  p.hchunks = p.lpt && a.cu_q == nullptr && (a.Hkv * a.B) % 16 == 0 ? 2 : 1;
  p.c = a.scale * kLog2e;
  p.B = a.B;
  dim3 grid(p.n_qtiles * a.Hq * a.B);
  hipLaunchKernelGGL((fwd_bf16_kernel<C>), grid, dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

// Tile-shape override for tuning (FA_FWD_VARIANT), read at every call.
int variant() {
  const char* e = getenv("FA_FWD_VARIANT");
  return e ? atoi(e) : 0;
}

}  // namespace

bool fwd_bf16_supported(int d) { return d == 64 || d == 128 || d == 256; }

// Tile shapes per head dimension, chosen by measurement on MI355X: d=64
// takes 64-key tiles at three waves per SIMD (128-key tiles at two measured
// 3.5% slower), d=128 64-key tiles at two waves per SIMD, d=256 32-key
// tiles at two waves per SIMD (without spills).
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64:
      switch (variant()) {
        case 1: return launch<Cfg<64, 64, 4, 2, 2, 2>>(a, stream);
        case 2: return launch<Cfg<64, 32, 4, 2, 2, 2>>(a, stream);
        case 3: return launch<Cfg<64, 64, 8, 1, 2, 2>>(a, stream);
        default: return launch<Cfg<64, 64, 4, 1, 2, 3>>(a, stream);
      }
    case 128:
      switch (variant()) {
        case 4: return launch<Cfg<128, 32, 2, 2, 4, 1, true>>(a, stream);
        // the hand-scheduled 64-row shape: parity-green, measured 5-11%
        // slower than the default (one wavefront per SIMD cannot issue the
        // softmax's vector work fast enough beside its MFMAs)
        case 5: return launch<Cfg<128, 64, 2, 2, 2, 1, false, true>>(a, stream);
        case 1: return launch<Cfg<128, 64, 8, 1, 2, 2>>(a, stream);
        case 2: return launch<Cfg<128, 32, 8, 1, 2, 2>>(a, stream);
        case 3: return launch<Cfg<128, 64, 8, 1, 3, 2>>(a, stream);
        default: return launch<Cfg<128, 64, 4, 1, 2, 2>>(a, stream);
      }
    case 256:
      switch (variant()) {
        case 1: return launch<Cfg<256, 64, 4, 1, 2, 1>>(a, stream);
        case 2: return launch<Cfg<256, 32, 4, 1, 3, 1>>(a, stream);
        default: return launch<Cfg<256, 32, 4, 1, 2, 2>>(a, stream);
      }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
