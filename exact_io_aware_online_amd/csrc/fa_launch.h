// fa_launch.h - host-side launchers behind the C ABI (internal).
//
// The C entry points in fa_api.cpp validate arguments and then call these;
// each launcher picks the kernel instantiation for the head dimension and
// enqueues it on the caller's stream. They assume validated arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, Hq, Hkv, Nq, Nk, d;
  int causal;  // top-left causal; the bf16 kernel reads the window fields below
  float scale;
  // key j is visible to query i iff i + off - window_left <= j <=
  // i + off + window_right (negative: unlimited), off = Nk_b - Nq_b when
  // bottom_right, else 0
  int window_left = -1, window_right = -1, bottom_right = 0;
  // packed variable-length batch (null: dense); Nq is then the longest
  // query sequence
  const int32_t* cu_q = nullptr;
  const int32_t* cu_k = nullptr;
  int total_q = 0, total_k = 0;
};

struct DecodeArgs {
  const void* q;
  const void* kcache;
  const void* vcache;
  const int32_t* seqlens;
  void* o;
  float* lse;  // may be null
  int num_splits;
  int B, Hq, Hkv, capacity, d;
  float scale;
  void* workspace;  // >= decode_workspace_bytes(...) when num_splits > 1
  // paged cache: null for a contiguous (B, capacity, Hkv, d) cache
  const int32_t* block_table = nullptr;
  int page_size = 0, pages_per_seq = 0, num_pages = 0;
  // Nq queries per sequence (q, o: (B, Nq, Hq, d); lse: (B, Hq, Nq)),
  // bottom-right causal when `causal`; k_new / v_new (B, Nq, Hkv, d), when
  // non-null, are written into the cache at rows seqlens[b] .. + Nq - 1
  // and attended
  int Nq = 1;
  int causal = 0;
  const void* k_new = nullptr;
  const void* v_new = nullptr;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Nq, Nk, d;  // packed batches: Nq, Nk are the longest sequences
  float scale;
  void* workspace;  // >= bwd_workspace_bytes(B, Hq, Nq)
  // visibility as in FwdArgs: i + off - window_left <= j <= i + off +
  // window_right, off = Nk_b - Nq_b when bottom_right (top-left causal:
  // window (-1, 0), bottom_right 0)
  int window_left = -1, window_right = -1, bottom_right = 0;
  const int32_t* cu_q = nullptr;  // packed variable-length batch, or null
  const int32_t* cu_k = nullptr;
  int total_q = 0, total_k = 0;
};

// FP8 (e4m3) forward: a bf16 tensor quantised per 64-row block of one
// (batch, head), optionally rotated first (signs non-null)
struct Fp8QuantArgs {
  const void* x;       // (B, N, H, d) bf16
  const float* signs;  // (d,) +-1, or null
  void* codes;         // (B, H, Np, d), or (B, H, d, Np) when transpose
  uint8_t* scales;     // (B, H, Np / 64) E8M0
  int transpose;
  int B, N, H, d;
};

struct Fp8FwdArgs {
  const void* q8;  // (B, Hq, Nqp, d) codes
  const uint8_t* q_scales;
  const void* k8;  // (B, Hkv, Nkp, d)
  const uint8_t* k_scales;
  const void* vt8;  // (B, Hkv, d, Nkp)
  const uint8_t* v_scales;
  void* o;     // (B, Nq, Hq, d) bf16
  float* lse;  // (B, Hq, Nq) or null
  int B, Hq, Hkv, Nq, Nk, d, causal;
  float scale;
};

constexpr int kFp8Block = 64;       // rows per quantisation block
constexpr int kFp8MaxKeys = 65536;  // keys per sequence the FP8 forward accepts
int fp8_padded_rows(int n);         // n rounded up to kFp8Block
bool fp8_quant_supported(int d);
bool fp8_fwd_supported(int d);
hipError_t launch_quant_fp8(const Fp8QuantArgs& a, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream);

// Keys per split for a cache of `capacity` rows cut into `num_splits`
// pieces: the smallest multiple of the decode key tile >= ceil(cap / S).
int decode_chunk(int capacity, int num_splits);
constexpr int kDecodePageAlign = 64;  // page sizes must be multiples of this
size_t decode_workspace_bytes(int B, int Hq, int d, int num_splits);
// Resident workgroups per CU of the balanced single-query decode kernel
// that a call with `pairs` (sequence, key/value head) pairs runs
// (decode_resident_per_cu) and of the split kernel that serves appends and
// several queries per sequence, for head dimension d (occupancy API; 2
// when no device can be queried).
int decode_resident_per_cu(int d, int64_t pairs);
int decode_split_resident_per_cu(int d);

bool fwd_bf16_supported(int d);
bool fwd_f32_supported(int d);
bool decode_supported(int d, int group);
bool bwd_supported(int d);
size_t bwd_workspace_bytes(int B, int Hq, int Nq);

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace fa
