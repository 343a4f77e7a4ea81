// fa_api.cpp - the C ABI declared in include/fa.h.
//
// Host-side shape policing before any launch (pyshine.com FlashAttention
// code tour, "Why You Need This" and the C++ layer described there, which
// validates strides and head dimensions and dispatches on head dimension).
// Every check runs before the first HIP call, so a rejected call touches
// neither the device nor the caller's buffers.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace fa {
// Defined beside the decode kernels: whether a split decode call of these
// sizes takes the balanced schedule.
bool decode_balanced(int B, int Nq, int Hq, int Hkv, bool append);
}  // namespace fa

namespace {

// Scratch of the allocation-free decode entry point: one copy per GPU in
// static device memory, resolved to a device address once per device.
__device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch` (looked up with that
// device current on its first use), or null if the lookup fails. Host code
// uses only this address: the array's own name is a host-side stand-in.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

constexpr int kAbiVersion = 2;

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

// Row counts (sequence lengths, capacities, packed totals) that the launch
// code rounds up to whole tiles in 32-bit integers: counts within 1024 of
// INT_MAX are rejected, so that rounding never overflows.
constexpr int kMaxRows = 0x7fffffff - 1023;
bool rows_ok(int n) { return n <= kMaxRows; }

// Device sizes given to the split policies, bounded so that their products
// stay far inside 64-bit range.
int clamp_count(int n, int hi) { return n > hi ? hi : n; }

fa_status_t launch_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

}  // namespace

extern "C" {

int fa_abi_version(void) { return kAbiVersion; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported head_dim/dtype/group/size";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    default: return "FA_ERR_UNKNOWN";
  }
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   int causal, float scale, int dtype, void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
  const bool supported = dtype == FA_DTYPE_BF16 ? fa::fwd_bf16_supported(d) : fa::fwd_f32_supported(d);
  if (!supported) return FA_ERR_UNSUPPORTED;
  // the prefill grid is one dimension of ceil(Nq / 64) * Hq * B workgroups at most
  if (Hq > 65535 || B > 65535 || (((int64_t)Nq + 63) / 64) * Hq * B > 0x7fffffff) return FA_ERR_UNSUPPORTED;
  // a sequence's first query and key rows are b Nq and b Nk (32-bit)
  if ((int64_t)B * Nq > 0x7fffffff || (int64_t)B * Nk > 0x7fffffff || !rows_ok(Nq) || !rows_ok(Nk))
    return FA_ERR_UNSUPPORTED;
  if (B == 0 || Nq == 0) return FA_OK;
  if (q == nullptr || o == nullptr) return FA_ERR_INVALID_ARG;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return FA_ERR_INVALID_ARG;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.causal = causal;
  a.scale = scale;
  a.window_left = -1;
  a.window_right = causal ? 0 : -1;
  a.bottom_right = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch_status(dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(a, s) : fa::launch_fwd_f32(a, s));
}

fa_status_t fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d,
                          int window_left, int window_right, float scale, void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (!fa::fwd_bf16_supported(d)) return FA_ERR_UNSUPPORTED;
  if (Hq > 65535 || B > 65535 || (((int64_t)Nq + 63) / 64) * Hq * B > 0x7fffffff) return FA_ERR_UNSUPPORTED;
  // a sequence's first query and key rows are b Nq and b Nk (32-bit)
  if ((int64_t)B * Nq > 0x7fffffff || (int64_t)B * Nk > 0x7fffffff || !rows_ok(Nq) || !rows_ok(Nk))
    return FA_ERR_UNSUPPORTED;
  if (B == 0 || Nq == 0) return FA_OK;
  if (q == nullptr || o == nullptr) return FA_ERR_INVALID_ARG;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.causal = 0;
  a.scale = scale;
  a.window_left = window_left < 0 ? -1 : window_left;
  a.window_right = window_right < 0 ? -1 : window_right;
  a.bottom_right = 1;
  return launch_status(fa::launch_fwd_bf16(a, static_cast<hipStream_t>(stream)));
}

fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int B, int Hq, int Hkv, int max_seqlen_q, int total_q, int total_k, int d,
                          int window_left, int window_right, float scale, void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || max_seqlen_q < 0 || total_q < 0 || total_k < 0 || d <= 0)
    return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (!fa::fwd_bf16_supported(d)) return FA_ERR_UNSUPPORTED;
  if (Hq > 65535 || B > 65535 || (((int64_t)max_seqlen_q + 63) / 64) * Hq * B > 0x7fffffff ||
      !rows_ok(max_seqlen_q) || !rows_ok(total_q) || !rows_ok(total_k))
    return FA_ERR_UNSUPPORTED;
  if (B == 0 || max_seqlen_q == 0 || total_q == 0) return FA_OK;
  if (q == nullptr || o == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return FA_ERR_INVALID_ARG;
  if (total_k > 0 && (k == nullptr || v == nullptr)) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = max_seqlen_q;
  a.Nk = 0;
  a.d = d;
  a.causal = 0;
  a.scale = scale;
  a.window_left = window_left < 0 ? -1 : window_left;
  a.window_right = window_right < 0 ? -1 : window_right;
  a.bottom_right = 1;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  return launch_status(fa::launch_fwd_bf16(a, static_cast<hipStream_t>(stream)));
}

size_t fa_fwd_kvcache_workspace_size(int B, int Hq, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || d <= 0 || num_splits <= 1) return 0;
  return fa::decode_workspace_bytes(B, Hq, d, num_splits);
}

namespace {

int current_cus() {
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
    return prop.multiProcessorCount;
  (void)hipGetLastError();
  return 256;
}

}  // namespace

int fa_kvcache_default_splits(int B, int Hkv, int capacity, int d, int num_cus, int wgs_per_cu) {
  if (B <= 0 || Hkv <= 0 || capacity <= 0) return 1;
  if (num_cus <= 0) num_cus = current_cus();
  if (wgs_per_cu <= 0) wgs_per_cu = fa::decode_resident_per_cu(d, (int64_t)B * Hkv);
  num_cus = clamp_count(num_cus, 1 << 16);
  wgs_per_cu = clamp_count(wgs_per_cu, 1 << 10);
  // The balanced decode runs (num_splits - 1) B Hkv equal runs of cache
  // tiles, each ideally on a resident workgroup of its own. Runs come in
  // waves of `slots`; a wave that holds few runs streams at a fraction of
  // the bandwidth. So take the fewest runs per pair whose waves leave at
  // most 1/8 of the slot-time idle (else the least idle), among 1 .. max(8,
  // slots / pairs) runs per pair, each run at least about 8 tiles of 64
  // keys long so its start is amortised. Measured on MI355X (GQA 32/8, d =
  // 128, lengths uniform over the upper seven eighths of the capacity): 48
  // pairs on 512 slots 30.6 us with 480 runs against 38.1 us with 528 (a
  // second wave of 16), 1088 pairs on 1024 slots 406 us with 5 runs per
  // pair against 482 us with one, 600 pairs 235 us with 3 runs per pair
  // against 257 us with one. With four or more pairs per resident slot, or
  // a cache of one tile, one pass per pair without a combine is as
  // balanced.
  const long slots = (long)num_cus * wgs_per_cu;
  const long pairs = (long)B * Hkv;
  const long tiles = ((long)capacity + 63) / 64;
  if (pairs >= 4 * slots || tiles <= 1) return 1;
  const long by_len = tiles / 8 > 1 ? tiles / 8 : 1;
  long kmax = slots / pairs > 8 ? slots / pairs : 8;
  if (kmax > by_len) kmax = by_len;
  if (kmax > 65534) kmax = 65534;
  long per_pair = 1, best_idle = 0, best_waves = 1;
  for (long k = 1; k <= kmax; ++k) {
    const long u = k * pairs, waves = (u + slots - 1) / slots;
    const long idle = waves * slots - u;  // slot-runs left idle by the last wave
    if (k == 1 || idle * best_waves < best_idle * waves) {
      per_pair = k;
      best_idle = idle;
      best_waves = waves;
    }
    if (8 * idle <= waves * slots) break;
  }
  long s = 1 + per_pair;
  if (s > 65535) s = 65535;
  return (int)s;
}

int fa_kvcache_append_default_splits(int B, int Nq, int Hkv, int Hq, int capacity, int d, int num_cus,
                                     int wgs_per_cu) {
  if (B <= 0 || Nq <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 || capacity <= 0) return 1;
  // Calls that take the balanced decode use its rule, the one-query rule.
  if (fa::decode_balanced(B, Nq, Hq, Hkv, true)) return fa_kvcache_default_splits(B, Hkv, capacity, d, num_cus, wgs_per_cu);
  if (num_cus <= 0) num_cus = current_cus();
  if (wgs_per_cu <= 0) wgs_per_cu = fa::decode_split_resident_per_cu(d);
  num_cus = clamp_count(num_cus, 1 << 16);
  wgs_per_cu = clamp_count(wgs_per_cu, 1 << 10);
  // Splits of about 1024 keys keep each split workgroup's stream long
  // enough to amortise its start (measured best on MI355X against 512 and
  // 768), and enough of them give every CU `wgs_per_cu` resident
  // workgroups; a workgroup serves 16 (query, query head) columns.
  const long groups = ((long)Nq * (Hq / Hkv) + 15) / 16;
  const long by_len = ((long)capacity + 1023) / 1024;
  // beyond about four waves of split workgroups the extra splits only add
  // partials and combine work (32 columns, B = 64, GQA 32/8, d = 128: 466 us
  // at 2 splits against 498 us at 8; 5 queries: 456 against 474 us); with
  // that many (sequence, KV head, column group) items already, one split
  // (the test avoids forming the possibly huge product)
  const long max_wgs = 4L * num_cus * wgs_per_cu;
  if (groups >= max_wgs || (long)B * Hkv > (max_wgs - 1) / groups) return 1;
  const long items = (long)B * Hkv * groups;
  const long by_fill = ((long)num_cus * wgs_per_cu + items - 1) / items;
  long s = by_len > by_fill ? by_len : by_fill;
  if (items * s > max_wgs) s = max_wgs / items;
  const long max_s = ((long)capacity + 63) / 64;  // at least one 64-key block per split
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 65535) s = 65535;
  return (int)s;
}

namespace {

fa_status_t kvcache(const void* q, const void* k_new, const void* v_new, const void* kcache, const void* vcache,
                    const int32_t* block_table, int page_size, int pages_per_seq, int num_pages,
                    const int32_t* cache_seqlens, void* o, float* lse, int causal,
                    int num_splits, int B, int Nq, int Hq, int Hkv, int capacity, int d,
                    float scale, void* workspace, size_t workspace_bytes, void* stream,
                    bool check_only = false) {
  if (B < 0 || Nq < 1 || Hq <= 0 || Hkv <= 0 || capacity < 0 || d <= 0 || num_splits < 1) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if ((k_new == nullptr) != (v_new == nullptr)) return FA_ERR_INVALID_ARG;
  if (!fa::decode_supported(d, Hq / Hkv)) return FA_ERR_UNSUPPORTED;
  if (num_splits > 65535 || Hkv > 65535 || B > 65535) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * Nq * Hq > 0x7fffffff || (int64_t)Nq * Hq > 0x7fffffff || !rows_ok(capacity) || !rows_ok(Nq))
    return FA_ERR_UNSUPPORTED;
  if (B == 0) return FA_OK;
  if (q == nullptr || o == nullptr || cache_seqlens == nullptr) return FA_ERR_INVALID_ARG;
  if (capacity > 0 && (kcache == nullptr || vcache == nullptr)) return FA_ERR_INVALID_ARG;
  if (check_only) return FA_OK;  // every check but the workspace's
  const size_t need = fa::decode_workspace_bytes(B * Nq, Hq, d, num_splits);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FA_ERR_WORKSPACE;

  fa::DecodeArgs a;
  a.q = q;
  a.kcache = kcache;
  a.vcache = vcache;
  a.seqlens = cache_seqlens;
  a.o = o;
  a.lse = lse;
  a.num_splits = num_splits;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.capacity = capacity;
  a.d = d;
  a.scale = scale;
  a.workspace = workspace;
  a.block_table = block_table;
  a.page_size = page_size;
  a.pages_per_seq = pages_per_seq;
  a.num_pages = num_pages;
  a.Nq = Nq;
  a.causal = causal != 0;
  a.k_new = k_new;
  a.v_new = v_new;
  return launch_status(fa::launch_decode(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

fa_status_t fa_fwd_kvcache(const void* q, const void* kcache, const void* vcache,
                           const int32_t* cache_seqlens, void* o, float* lse,
                           int num_splits, int B, int Hq, int Hkv, int capacity, int d,
                           float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return kvcache(q, nullptr, nullptr, kcache, vcache, nullptr, 0, 0, 0, cache_seqlens, o, lse, 0, num_splits, B, 1,
                 Hq, Hkv, capacity, d, scale, workspace, workspace_bytes, stream);
}

fa_status_t fa_fwd_kvcache_noalloc(const void* q, const void* kcache, const void* vcache,
                                   const int32_t* cache_seqlens, void* o, float* lse,
                                   int num_splits, int B, int Hq, int Hkv, int capacity, int d,
                                   float scale, void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || capacity < 0 || d <= 0 || num_splits < 1) return FA_ERR_INVALID_ARG;
  const size_t need = B > 0 ? fa::decode_workspace_bytes(B, Hq, d, num_splits) : 0;
  if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    // the argument checks come first: a call they reject must not touch the device
    const fa_status_t st = kvcache(q, nullptr, nullptr, kcache, vcache, nullptr, 0, 0, 0, cache_seqlens, o, lse, 0,
                                   num_splits, B, 1, Hq, Hkv, capacity, d, scale, nullptr, 0, nullptr, true);
    if (st != FA_OK) return st;
    ws = scratch_on_current_device();
    if (ws == nullptr) return FA_ERR_LAUNCH;
  }
  return kvcache(q, nullptr, nullptr, kcache, vcache, nullptr, 0, 0, 0, cache_seqlens, o, lse, 0, num_splits, B, 1,
                 Hq, Hkv, capacity, d, scale, ws, need, stream);
}

fa_status_t fa_fwd_kvcache_append(const void* q, const void* k_new, const void* v_new, void* kcache, void* vcache,
                                  const int32_t* cache_seqlens, void* o, float* lse, int causal, int num_splits,
                                  int B, int Nq, int Hq, int Hkv, int capacity, int d, float scale,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return kvcache(q, k_new, v_new, kcache, vcache, nullptr, 0, 0, 0, cache_seqlens, o, lse, causal, num_splits, B, Nq,
                 Hq, Hkv, capacity, d, scale, workspace, workspace_bytes, stream);
}

fa_status_t fa_fwd_kvcache_paged(const void* q, const void* kpages, const void* vpages,
                                 const int32_t* block_table, const int32_t* cache_seqlens, void* o, float* lse,
                                 int num_splits, int B, int Hq, int Hkv, int page_size, int pages_per_seq,
                                 int num_pages, int d, float scale, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (page_size <= 0 || page_size % fa::kDecodePageAlign != 0 || pages_per_seq <= 0 || num_pages <= 0)
    return FA_ERR_INVALID_ARG;
  if ((int64_t)page_size * pages_per_seq > kMaxRows) return FA_ERR_UNSUPPORTED;
  if (B > 0 && block_table == nullptr) return FA_ERR_INVALID_ARG;
  return kvcache(q, nullptr, nullptr, kpages, vpages, block_table, page_size, pages_per_seq, num_pages, cache_seqlens,
                 o, lse, 0, num_splits, B, 1, Hq, Hkv, page_size * pages_per_seq, d, scale, workspace,
                 workspace_bytes, stream);
}

fa_status_t fa_fwd_kvcache_paged_append(const void* q, const void* k_new, const void* v_new, void* kpages,
                                        void* vpages, const int32_t* block_table, const int32_t* cache_seqlens,
                                        void* o, float* lse, int causal, int num_splits, int B, int Nq, int Hq,
                                        int Hkv, int page_size, int pages_per_seq, int num_pages, int d, float scale,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (page_size <= 0 || page_size % fa::kDecodePageAlign != 0 || pages_per_seq <= 0 || num_pages <= 0)
    return FA_ERR_INVALID_ARG;
  if ((int64_t)page_size * pages_per_seq > kMaxRows) return FA_ERR_UNSUPPORTED;
  if (B > 0 && block_table == nullptr) return FA_ERR_INVALID_ARG;
  return kvcache(q, k_new, v_new, kpages, vpages, block_table, page_size, pages_per_seq, num_pages, cache_seqlens, o,
                 lse, causal, num_splits, B, Nq, Hq, Hkv, page_size * pages_per_seq, d, scale, workspace,
                 workspace_bytes, stream);
}

int fa_fp8_padded_rows(int n) { return n <= 0 || !rows_ok(n) ? 0 : fa::fp8_padded_rows(n); }

fa_status_t fa_quantize_fp8(const void* x, const float* signs, void* codes, uint8_t* scales, int transpose,
                            int B, int N, int H, int d, void* stream) {
  if (B < 0 || N < 0 || H <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (transpose != 0 && transpose != 1) return FA_ERR_INVALID_ARG;
  if (!fa::fp8_quant_supported(d)) return FA_ERR_UNSUPPORTED;
  if (B > 65535 || H > 65535 || N > 0x7fffffff - 64) return FA_ERR_UNSUPPORTED;
  if (B == 0 || N == 0) return FA_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return FA_ERR_INVALID_ARG;
  fa::Fp8QuantArgs a;
  a.x = x;
  a.signs = signs;
  a.codes = codes;
  a.scales = scales;
  a.transpose = transpose;
  a.B = B;
  a.N = N;
  a.H = H;
  a.d = d;
  return launch_status(fa::launch_quant_fp8(a, static_cast<hipStream_t>(stream)));
}

fa_status_t fa_fwd_fp8(const void* q8, const uint8_t* q_scales, const void* k8, const uint8_t* k_scales,
                       const void* vt8, const uint8_t* v_scales, void* o, float* lse,
                       int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale, void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (!fa::fp8_fwd_supported(d)) return FA_ERR_UNSUPPORTED;
  if (Nk > fa::kFp8MaxKeys || Nq > 0x7fffffff - 128) return FA_ERR_UNSUPPORTED;
  if (Hq > 65535 || B > 65535 || (((int64_t)Nq + 127) / 128) * Hq * B > 0x7fffffff) return FA_ERR_UNSUPPORTED;
  if (B == 0 || Nq == 0) return FA_OK;
  if (q8 == nullptr || q_scales == nullptr || o == nullptr) return FA_ERR_INVALID_ARG;
  if (Nk > 0 && (k8 == nullptr || k_scales == nullptr || vt8 == nullptr || v_scales == nullptr))
    return FA_ERR_INVALID_ARG;
  fa::Fp8FwdArgs a;
  a.q8 = q8;
  a.q_scales = q_scales;
  a.k8 = k8;
  a.k_scales = k_scales;
  a.vt8 = vt8;
  a.v_scales = v_scales;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.causal = causal;
  a.scale = scale;
  return launch_status(fa::launch_fwd_fp8(a, static_cast<hipStream_t>(stream)));
}

size_t fa_bwd_workspace_size(int B, int Hq, int Nq) {
  if (B <= 0 || Hq <= 0 || Nq <= 0) return 0;
  return fa::bwd_workspace_bytes(B, Hq, Nq);
}

namespace {

// Shared checks and dispatch of the three backward entry points. Nq and Nk
// are the (longest) sequence lengths; for a packed batch total_q / total_k
// are the packed row counts and cu_q / cu_k the sequence offsets.
fa_status_t bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, const int32_t* cu_q, const int32_t* cu_k, int B, int Hq, int Hkv,
                int Nq, int Nk, int total_q, int total_k, int d, int window_left, int window_right,
                int bottom_right, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const bool packed = cu_q != nullptr || cu_k != nullptr;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || d <= 0 || total_q < 0 || total_k < 0)
    return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (!fa::bwd_supported(d)) return FA_ERR_UNSUPPORTED;
  // one-dimensional grids, and the workspace addressed with 32-bit offsets
  const int64_t nq_pad = ((int64_t)Nq + 31) / 32 * 32;
  if (Hq > 65535 || B > 65535 || (((int64_t)Nq + 127) / 128) * Hq * B > 0x7fffffff ||
      (((int64_t)Nk + 127) / 128) * Hkv * B > 0x7fffffff || 2 * (int64_t)B * Hq * nq_pad * 4 > 0xffffffffLL)
    return FA_ERR_UNSUPPORTED;
  const int64_t rows_q = packed ? total_q : (int64_t)B * Nq;
  const int64_t rows_k = packed ? total_k : (int64_t)B * Nk;
  if (rows_q > 0x7fffffff || rows_k > 0x7fffffff) return FA_ERR_UNSUPPORTED;  // 32-bit row indices
  if (!rows_ok(Nq) || !rows_ok(Nk) || !rows_ok(total_q) || !rows_ok(total_k)) return FA_ERR_UNSUPPORTED;
  if (B == 0 || (rows_q == 0 && rows_k == 0)) return FA_OK;
  if (packed && (cu_q == nullptr || cu_k == nullptr)) return FA_ERR_INVALID_ARG;
  if (rows_q > 0 && (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr || dq == nullptr))
    return FA_ERR_INVALID_ARG;
  if (rows_k > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)) return FA_ERR_INVALID_ARG;
  const size_t need = Nq > 0 ? fa::bwd_workspace_bytes(B, Hq, Nq) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FA_ERR_WORKSPACE;

  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.scale = scale;
  a.workspace = workspace;
  a.window_left = window_left < 0 ? -1 : window_left;
  a.window_right = window_right < 0 ? -1 : window_right;
  a.bottom_right = bottom_right;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.total_q = total_q;
  a.total_k = total_k;
  return launch_status(fa::launch_bwd(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return bwd(q, k, v, o, lse, dout, dq, dk, dv, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, 0, 0, d, -1, causal ? 0 : -1, 0,
             scale, workspace, workspace_bytes, stream);
}

fa_status_t fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, int window_left, int window_right,
                          float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd(q, k, v, o, lse, dout, dq, dk, dv, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, 0, 0, d, window_left,
             window_right, 1, scale, workspace, workspace_bytes, stream);
}

fa_status_t fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int B, int Hq, int Hkv, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                          int d, int window_left, int window_right, float scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)) return FA_ERR_INVALID_ARG;
  return bwd(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, max_seqlen_q, max_seqlen_k,
             total_q, total_k, d, window_left, window_right, 1, scale, workspace, workspace_bytes, stream);
}

}  // extern "C"
