// fa_kernels.h -- host-side launch interface of the attention kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Compute units of a whole MI355X.  Launch heuristics use the current
// device's count (device_cu_count); this is its value when no device answers.
constexpr int kFullChipCUs = 256;

// Compute units of the current device (hipDeviceAttributeMultiprocessorCount),
// or kFullChipCUs if the query fails.  One HIP runtime query per call.
int device_cu_count();

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  bool causal;
  int dtype;  // enum fa_dtype
  // Packed batch: cumulative query / key counts [B + 1] (device), token
  // totals; Nq and Nk then bound the sequence lengths.  Null for dense.
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int tot_q = 0, tot_k = 0;
  // Paged KV cache (k, v are [num_blocks, Hkv, 16, d] page caches): block
  // table [B, max_blocks] and cached tokens per sequence [B] (device).  Null
  // for contiguous K, V.
  const int* block_table = nullptr;
  const int* seq_lens = nullptr;
  int max_blocks = 0, num_blocks = 0;
  // Compute units of the device the launch runs on (sizes the work-groups).
  int cus = kFullChipCUs;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;  // workspace: -D_i = -sum_c dO_ic O_ic (one per query row), then LSE_i*log2(e)
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  bool causal;
  int dtype;
  const int* cu_q = nullptr;  // packed batch, as in FwdArgs
  const int* cu_k = nullptr;
  int tot_q = 0, tot_k = 0;
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int* block_table;
  const int* seq_lens;
  void* o;
  float* lse;  // may be null
  float* part; // workspace: [B, Hq, splits, d + 4] float32
  int B, Hq, Hkv, d, block_size, max_blocks, num_blocks, splits;
  float scale;
  int dtype;
};

// FP8 (E4M3) forward: q, k, v are E4M3 codes, o is bf16; workspace holds
// the staged Vᵀ tiles (fp8_vt_bytes).
struct Fp8FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  void* workspace;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale, q_descale, k_descale, v_descale;
  bool causal;
};

// The exponent scale c = scale * log2(e) (times the FP8 descales) as the
// forward kernels take it: its magnitude, with a zero scale replaced by 2^-100
// (every exponential then rounds to 1, as exp(0) would), and whether it is
// negative (the kernels then flip the sign of Q, or of K in the dK/dV kernel,
// which is exact, so that the row max of c*s is c times the max of s).  Worked out on the host so that the
// kernels keep c in a scalar register.
struct ExpScale {
  float c;
  int neg_q;
};
inline ExpScale exp_scale(float c) { return ExpScale{c < 0.f ? -c : (c > 0.f ? c : 0x1p-100f), c < 0.f ? 1 : 0}; }

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// The forward whose two wave groups split each 128-row query tile's keys
// (16-bit types; dense, packed or paged K/V; used for short grids).
hipError_t launch_fwd_keysplit(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream);
size_t fp8_vt_bytes(int B, int Hkv, int Nk, int d);
// Backward phases (bit mask); kBwdAll runs them in order on one stream.
// kBwdDqRowTerms is the dQ phase computing the row terms itself (in place of
// kBwdPrep); with kBwdDkdv it runs first and dK/dV after it, and kBwdFused is
// that pair, the whole backward in two kernels.
constexpr int kBwdPrep = 1, kBwdDkdv = 2, kBwdDq = 4, kBwdAll = 7, kBwdDqRowTerms = 8;
constexpr int kBwdFused = kBwdDqRowTerms | kBwdDkdv;
hipError_t launch_bwd(const BwdArgs& a, int phases, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Size of the fixed scratch area of the allocation-free decode (one per GPU).
constexpr size_t kDecodeScratchBytes = (size_t)8 << 20;
// Device address of the current device's scratch area (resolved once per
// device, then cached).  The only HIP calls are hipGetDevice and, on a
// device's first use, hipGetSymbolAddress.
hipError_t decode_scratch_area(void** out);

}  // namespace fa
