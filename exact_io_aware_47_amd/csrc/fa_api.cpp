// fa_api.cpp -- C ABI of the attention library: argument validation (host
// only, before any HIP call), workspace sizing and kernel dispatch.
#include "flash_attn.h"

#include <math.h>
#include <stdint.h>

#include "fa_kernels.h"

static_assert(fa::kDecodeScratchBytes == FLASH_ATTN_DECODE_SCRATCH_BYTES, "scratch size out of sync with the header");

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;  // per tensor, keeps 32-bit element offsets valid
constexpr int kMaxDecodeSplits = 1 << 16;        // explicit decode split counts above this are refused

int elem_bytes(int dtype) { return dtype == FA_F32 ? 4 : 2; }
bool dtype_ok(int dtype) { return dtype == FA_F32 || dtype == FA_F16 || dtype == FA_BF16; }
bool headdim_ok(int d) { return d == 32 || d == 64 || d == 128; }

// Shared checks of the dense entry points, in the documented order.
int check_dense(int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int dtype) {
  if (!dtype_ok(dtype)) return FA_ERR_DTYPE;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_SHAPE;
  if (!headdim_ok(d)) return FA_ERR_HEADDIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  if ((int64_t)B * Hq * Nq * d >= kMaxElems || (int64_t)B * Hkv * Nk * d >= kMaxElems) return FA_ERR_SHAPE;
  // One (batch, head) slab is addressed with 32-bit byte offsets.
  if ((int64_t)Nq * d * elem_bytes(dtype) >= kMaxElems || (int64_t)Nk * d * elem_bytes(dtype) >= kMaxElems)
    return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

// Checks of the packed (variable-length) entry points, in the documented order.
int check_varlen(int B, int Hq, int Hkv, int total_q, int total_k, int max_q, int max_k, int d, float scale,
                 int dtype) {
  if (!dtype_ok(dtype)) return FA_ERR_DTYPE;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0 || max_q > total_q ||
      max_k > total_k)
    return FA_ERR_SHAPE;
  if (!headdim_ok(d)) return FA_ERR_HEADDIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  if ((int64_t)Hq * total_q * d >= kMaxElems || (int64_t)Hkv * total_k * d >= kMaxElems) return FA_ERR_SHAPE;
  // One (sequence, head) slab is addressed with 32-bit byte offsets.
  if ((int64_t)max_q * d * elem_bytes(dtype) >= kMaxElems || (int64_t)max_k * d * elem_bytes(dtype) >= kMaxElems)
    return FA_ERR_SHAPE;
  // Grids span (sequence, head, tile of the longest sequence); keep them and B + 1 in 32 bits.
  if ((int64_t)B * Hq * ((max_q + 127) / 128 + 1) >= kMaxElems ||
      (int64_t)B * Hkv * ((max_k + 127) / 128 + 1) >= kMaxElems)
    return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int launch_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* flash_attn_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid size (non-positive, or tensor too large)";
    case FA_ERR_HEADDIM: return "head dimension must be 32, 64 or 128";
    case FA_ERR_DTYPE: return "dtype must be FA_F32, FA_F16 or FA_BF16";
    case FA_ERR_GQA: return "Hq must be a multiple of Hkv";
    case FA_ERR_BLOCKSIZE: return "KV cache page size must be 16 tokens";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_ALIGN: return "a tensor pointer is misaligned (16 bytes; LSE and int32 arrays 4 bytes)";
    case FA_ERR_SCRATCH: return "the call needs more than the fixed scratch area of the allocation-free decode";
  }
  return "unknown error code";
}

int flash_attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq, int Hkv,
                   int Nq, int Nk, int d, float scale, int causal, int dtype, void* stream) {
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
  const int st = check_dense(B, Hq, Hkv, Nq, Nk, d, scale, dtype);
  if (st != FA_OK) return st;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4))
    return FA_ERR_ALIGN;
  fa::FwdArgs a;
  a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.d = d;
  a.scale = scale; a.causal = causal != 0; a.dtype = dtype;
  a.cus = fa::device_cu_count();
  return launch_status(fa::launch_fwd(a, (hipStream_t)stream));
}

int flash_attn_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE, const int* cu_seqlens_q,
                          const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                          int max_seqlen_k, int d, float scale, int causal, int dtype, void* stream) {
  if (!Q || !K || !V || !O || !LSE || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  const int st = check_varlen(B, Hq, Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d, scale, dtype);
  if (st != FA_OK) return st;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return FA_ERR_ALIGN;
  fa::FwdArgs a;
  a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = max_seqlen_q; a.Nk = max_seqlen_k; a.d = d;
  a.scale = scale; a.causal = causal != 0; a.dtype = dtype;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k; a.tot_q = total_q; a.tot_k = total_k;
  a.cus = fa::device_cu_count();
  return launch_status(fa::launch_fwd(a, (hipStream_t)stream));
}

size_t flash_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d, int dtype) {
  if (check_dense(B, Hq, Hkv, Nq, Nk, d, 1.0f, dtype) != FA_OK) return 0;
  return 2 * (size_t)B * Hq * Nq * sizeof(float);  // D row terms, then LSE * log2(e)
}

}  // extern "C"

namespace {

// Everything a backward phase may touch; unused pointers are NULL.
struct BwdPtrs {
  const void *Q, *K, *V, *O, *dO;
  const float* LSE;
  void *dQ, *dK, *dV;
  const void* workspace;
};

int run_bwd(const BwdPtrs& t, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
            size_t workspace_bytes, int phases, void* stream) {
  const int st = check_dense(B, Hq, Hkv, Nq, Nk, d, scale, dtype);
  if (st != FA_OK) return st;
  if (!t.workspace || workspace_bytes < flash_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, dtype))
    return FA_ERR_WORKSPACE;
  const void* dense[] = {t.Q, t.K, t.V, t.O, t.dO, t.dQ, t.dK, t.dV, t.workspace};
  for (const void* p : dense)
    if (p && !aligned(p, 16)) return FA_ERR_ALIGN;
  if (t.LSE && !aligned(t.LSE, 4)) return FA_ERR_ALIGN;
  fa::BwdArgs a;
  a.q = t.Q; a.k = t.K; a.v = t.V; a.o = t.O; a.dout = t.dO; a.lse = t.LSE;
  a.dq = t.dQ; a.dk = t.dK; a.dv = t.dV; a.dsum = (float*)t.workspace;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.d = d;
  a.scale = scale; a.causal = causal != 0; a.dtype = dtype;
  return launch_status(fa::launch_bwd(a, phases, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int flash_attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                   void* dQ, void* dK, void* dV, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                   int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA_ERR_NULL;
  const BwdPtrs t = {Q, K, V, O, dO, LSE, dQ, dK, dV, workspace};
  return run_bwd(t, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, workspace_bytes, fa::kBwdFused, stream);
}

int flash_attn_bwd_preprocess(const void* O, const void* dO, const float* LSE, int B, int Hq, int Nq, int d,
                              int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!O || !dO || !LSE) return FA_ERR_NULL;
  const BwdPtrs t = {nullptr, nullptr, nullptr, O, dO, LSE, nullptr, nullptr, nullptr, workspace};
  return run_bwd(t, B, Hq, Hq, Nq, Nq, d, 1.0f, 0, dtype, workspace_bytes, fa::kBwdPrep, stream);
}

int flash_attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO, void* dK, void* dV, int B,
                        int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
                        const void* workspace, size_t workspace_bytes, void* stream) {
  if (!Q || !K || !V || !dO || !dK || !dV) return FA_ERR_NULL;
  const BwdPtrs t = {Q, K, V, nullptr, dO, nullptr, nullptr, dK, dV, workspace};
  return run_bwd(t, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, workspace_bytes, fa::kBwdDkdv, stream);
}

int flash_attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO, void* dQ, int B, int Hq, int Hkv,
                      int Nq, int Nk, int d, float scale, int causal, int dtype, const void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!Q || !K || !V || !dO || !dQ) return FA_ERR_NULL;
  const BwdPtrs t = {Q, K, V, nullptr, dO, nullptr, dQ, nullptr, nullptr, workspace};
  return run_bwd(t, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, workspace_bytes, fa::kBwdDq, stream);
}

int flash_attn_bwd_dq_rowterms(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                               const float* LSE, void* dQ, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                               float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ) return FA_ERR_NULL;
  const BwdPtrs t = {Q, K, V, O, dO, LSE, dQ, nullptr, nullptr, workspace};
  return run_bwd(t, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, workspace_bytes, fa::kBwdDqRowTerms, stream);
}

size_t flash_attn_bwd_varlen_workspace_bytes(int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                                             int max_seqlen_k, int d, int dtype) {
  if (check_varlen(B, Hq, Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d, 1.0f, dtype) != FA_OK) return 0;
  return 2 * (size_t)Hq * total_q * sizeof(float);  // D row terms, then LSE * log2(e)
}

int flash_attn_bwd_varlen(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                          const float* LSE, void* dQ, void* dK, void* dV, const int* cu_seqlens_q,
                          const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                          int max_seqlen_k, int d, float scale, int causal, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV || !cu_seqlens_q || !cu_seqlens_k)
    return FA_ERR_NULL;
  const int st = check_varlen(B, Hq, Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d, scale, dtype);
  if (st != FA_OK) return st;
  const size_t need = flash_attn_bwd_varlen_workspace_bytes(B, Hq, Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k,
                                                            d, dtype);
  if ((need > 0 && !workspace) || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const void* dense[] = {Q, K, V, O, dO, dQ, dK, dV, workspace};
  for (const void* p : dense)
    if (p && !aligned(p, 16)) return FA_ERR_ALIGN;
  if (!aligned(LSE, 4) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4)) return FA_ERR_ALIGN;
  fa::BwdArgs a;
  a.q = Q; a.k = K; a.v = V; a.o = O; a.dout = dO; a.lse = LSE;
  a.dq = dQ; a.dk = dK; a.dv = dV; a.dsum = (float*)workspace;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = max_seqlen_q; a.Nk = max_seqlen_k; a.d = d;
  a.scale = scale; a.causal = causal != 0; a.dtype = dtype;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k; a.tot_q = total_q; a.tot_k = total_k;
  return launch_status(fa::launch_bwd(a, fa::kBwdFused, (hipStream_t)stream));
}

int flash_attn_prefill_paged(const void* Q, const void* K_cache, const void* V_cache, const int* block_table,
                             const int* seq_lens, void* O, float* LSE, int B, int Hq, int Hkv, int Nq, int d,
                             int block_size, int max_blocks_per_seq, int num_blocks, float scale, int causal, int dtype,
                             void* stream) {
  if (!Q || !K_cache || !V_cache || !block_table || !seq_lens || !O || !LSE) return FA_ERR_NULL;
  if (!dtype_ok(dtype)) return FA_ERR_DTYPE;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0) return FA_ERR_SHAPE;
  if (!headdim_ok(d)) return FA_ERR_HEADDIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  if (block_size != 16) return FA_ERR_BLOCKSIZE;
  if ((int64_t)B * Hq * Nq * d >= kMaxElems || (int64_t)Nq * d * elem_bytes(dtype) >= kMaxElems ||
      (int64_t)B * max_blocks_per_seq >= kMaxElems || (int64_t)max_blocks_per_seq * block_size >= kMaxElems)
    return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (!aligned(Q, 16) || !aligned(K_cache, 16) || !aligned(V_cache, 16) || !aligned(O, 16) || !aligned(LSE, 4) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return FA_ERR_ALIGN;
  fa::FwdArgs a;
  a.q = Q; a.k = K_cache; a.v = V_cache; a.o = O; a.lse = LSE;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = max_blocks_per_seq * block_size; a.d = d;
  a.scale = scale; a.causal = causal != 0; a.dtype = dtype;
  a.block_table = block_table; a.seq_lens = seq_lens; a.max_blocks = max_blocks_per_seq; a.num_blocks = num_blocks;
  a.cus = fa::device_cu_count();
  return launch_status(fa::launch_fwd(a, (hipStream_t)stream));
}

size_t flash_attn_fwd_fp8_workspace_bytes(int B, int Hkv, int Nk, int d) {
  if (B <= 0 || Hkv <= 0 || Nk <= 0 || (d != 64 && d != 128)) return 0;
  return fa::fp8_vt_bytes(B, Hkv, Nk, d);
}

int flash_attn_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq, int Hkv,
                       int Nq, int Nk, int d, float scale, float q_descale, float k_descale, float v_descale,
                       int causal, void* workspace, size_t workspace_bytes, void* stream) {
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  // Element counts and 32-bit byte offsets of the slabs (bf16 O is the widest),
  // and the pre-pass grid's second dimension.
  if ((int64_t)B * Hq * Nq * d >= kMaxElems || (int64_t)B * Hkv * (Nk + 63) / 64 * 64 * d >= kMaxElems ||
      (int64_t)Nq * d * 2 >= kMaxElems || (int64_t)(Nk + 63) / 64 * 64 * d >= kMaxElems || (int64_t)B * Hkv > 65535)
    return FA_ERR_SHAPE;
  if (!isfinite(scale) || !isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale) ||
      !isfinite(scale * q_descale * k_descale))
    return FA_ERR_SCALE;
  if (!workspace || workspace_bytes < flash_attn_fwd_fp8_workspace_bytes(B, Hkv, Nk, d)) return FA_ERR_WORKSPACE;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4) ||
      !aligned(workspace, 16))
    return FA_ERR_ALIGN;
  fa::Fp8FwdArgs a;
  a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE; a.workspace = workspace;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.d = d;
  a.scale = scale; a.q_descale = q_descale; a.k_descale = k_descale; a.v_descale = v_descale;
  a.causal = causal != 0;
  return launch_status(fa::launch_fwd_fp8(a, (hipStream_t)stream));
}

int flash_attn_decode_num_splits(int B, int Hkv, int max_blocks_per_seq, int block_size) {
  if (B <= 0 || Hkv <= 0 || max_blocks_per_seq <= 0 || block_size != 16) return 0;
  // Aim for 4 splits (waves) per compute unit of the current device, with at
  // least 4 pages per split: measured on the 32768-token decode (256 compute
  // units), 16 splits per sequence and K/V head beat 8, 32 and 64.
  const int64_t units = (int64_t)B * Hkv;
  int64_t splits = (4 * (int64_t)fa::device_cu_count() + units - 1) / units;
  const int64_t max_splits = max_blocks_per_seq / 4 > 0 ? max_blocks_per_seq / 4 : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return (int)splits;
}

size_t flash_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int max_blocks_per_seq, int block_size,
                                         int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !headdim_ok(d) || max_blocks_per_seq <= 0 ||
      block_size != 16 || num_splits < 0 || num_splits > kMaxDecodeSplits)
    return 0;
  const int splits = num_splits > 0 ? num_splits : flash_attn_decode_num_splits(B, Hkv, max_blocks_per_seq, block_size);
  return (size_t)B * Hq * splits * (d + 4) * sizeof(float);  // [O (d), m, l, 2 pad] per split
}

}  // extern "C"

namespace {

// Checks shared by the two decode entry points, in the documented order up to
// (not including) the workspace; on success *splits is the split count.
int check_decode(const void* Q, const void* K_cache, const void* V_cache, const int* block_table,
                 const int* seq_lens, const void* O, int B, int Hq, int Hkv, int d, int block_size,
                 int max_blocks_per_seq, int num_blocks, float scale, int num_splits, int dtype, int* splits) {
  if (!Q || !K_cache || !V_cache || !block_table || !seq_lens || !O) return FA_ERR_NULL;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || num_splits < 0)
    return FA_ERR_SHAPE;
  if (!headdim_ok(d)) return FA_ERR_HEADDIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  if (block_size != 16) return FA_ERR_BLOCKSIZE;
  // The split kernel's grid is (work-groups per (sequence, K/V head), B * Hkv):
  // its second dimension stays within 65535, and the split count within
  // kMaxDecodeSplits so that the first cannot overflow.
  if ((int64_t)B * max_blocks_per_seq >= kMaxElems || (int64_t)max_blocks_per_seq * block_size >= kMaxElems ||
      (int64_t)B * Hq * d >= kMaxElems || (int64_t)B * Hkv > 65535 || num_splits > kMaxDecodeSplits)
    return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  *splits = num_splits > 0 ? num_splits : flash_attn_decode_num_splits(B, Hkv, max_blocks_per_seq, block_size);
  return FA_OK;
}

bool decode_ptrs_aligned(const void* Q, const void* K_cache, const void* V_cache, const int* block_table,
                         const int* seq_lens, const void* O, const float* LSE) {
  return aligned(Q, 16) && aligned(K_cache, 16) && aligned(V_cache, 16) && aligned(O, 16) &&
         aligned(block_table, 4) && aligned(seq_lens, 4) && aligned(LSE, 4);
}

int run_decode(const void* Q, const void* K_cache, const void* V_cache, const int* block_table, const int* seq_lens,
               void* O, float* LSE, int B, int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
               int num_blocks, float scale, int splits, int dtype, void* part, void* stream) {
  fa::DecodeArgs a;
  a.q = Q; a.k_cache = K_cache; a.v_cache = V_cache; a.block_table = block_table; a.seq_lens = seq_lens;
  a.o = O; a.lse = LSE; a.part = (float*)part;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.block_size = block_size; a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks; a.splits = splits; a.scale = scale; a.dtype = dtype;
  return launch_status(fa::launch_decode(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int flash_attn_decode_paged(const void* Q, const void* K_cache, const void* V_cache, const int* block_table,
                            const int* seq_lens, void* O, float* LSE, int B, int Hq, int Hkv, int d, int block_size,
                            int max_blocks_per_seq, int num_blocks, float scale, int num_splits, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  int splits = 0;
  const int st = check_decode(Q, K_cache, V_cache, block_table, seq_lens, O, B, Hq, Hkv, d, block_size,
                              max_blocks_per_seq, num_blocks, scale, num_splits, dtype, &splits);
  if (st != FA_OK) return st;
  if (!workspace ||
      workspace_bytes < flash_attn_decode_workspace_bytes(B, Hq, Hkv, d, max_blocks_per_seq, block_size, splits))
    return FA_ERR_WORKSPACE;
  if (!decode_ptrs_aligned(Q, K_cache, V_cache, block_table, seq_lens, O, LSE) || !aligned(workspace, 16))
    return FA_ERR_ALIGN;
  return run_decode(Q, K_cache, V_cache, block_table, seq_lens, O, LSE, B, Hq, Hkv, d, block_size,
                    max_blocks_per_seq, num_blocks, scale, splits, dtype, workspace, stream);
}

int flash_attn_decode_paged_noalloc(const void* Q, const void* K_cache, const void* V_cache, const int* block_table,
                                    const int* seq_lens, void* O, float* LSE, int B, int Hq, int Hkv, int d,
                                    int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                                    int num_splits, int dtype, void* stream) {
  int splits = 0;
  const int st = check_decode(Q, K_cache, V_cache, block_table, seq_lens, O, B, Hq, Hkv, d, block_size,
                              max_blocks_per_seq, num_blocks, scale, num_splits, dtype, &splits);
  if (st != FA_OK) return st;
  if (flash_attn_decode_workspace_bytes(B, Hq, Hkv, d, max_blocks_per_seq, block_size, splits) >
      FLASH_ATTN_DECODE_SCRATCH_BYTES)
    return FA_ERR_SCRATCH;
  if (!decode_ptrs_aligned(Q, K_cache, V_cache, block_table, seq_lens, O, LSE)) return FA_ERR_ALIGN;
  void* part = nullptr;
  if (fa::decode_scratch_area(&part) != hipSuccess) return FA_ERR_LAUNCH;
  return run_decode(Q, K_cache, V_cache, block_table, seq_lens, O, LSE, B, Hq, Hkv, d, block_size,
                    max_blocks_per_seq, num_blocks, scale, splits, dtype, part, stream);
}

}  // extern "C"
