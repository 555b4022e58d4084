// fa_decode.hip -- split-KV decode over a paged KV cache for gfx950.
//
// FlashDecoding and PagedAttention as the tutorial "FlashAttention and
// efficient attention kernels" describes them ("Variant family"): the KV
// sequence of each new token is cut into splits whose partial softmax results
// are computed in parallel and reduced afterwards, and the keys/values are
// read from fixed-size pages reached through a block table.  Grouped-query
// heads follow the related-work page's paper #6: the query heads of one group
// share a K/V head, so they are processed together against each page.
//
// decode_split: every wave is one split of one (sequence, K/V head, group of
//   up to 16 query heads).  It walks its pages two at a time, double-buffered
//   (bounds-checked loads, one descriptor per page, so token slots past the
//   sequence end read as zero): K goes straight into registers in the A
//   operand layout of the score product, V through a private LDS ring for
//   the transposing reads.  Keeping K out of LDS halves the ring, so two
//   work-groups fit on a compute unit and twice the pages are in flight:
//     Sᵀ = K_page Qᵀ          (16 tokens x 16 query heads, 16x16x32 MFMA)
//     online softmax per query head (running max m, running sum l, log2 domain)
//     Oᵀ = Oᵀ exp2(m_old - m_new) + Vᵀ Pᵀ   (32 tokens per product; Vᵀ comes
//                                           from transposing LDS reads)
//   and writes its partial (Oᵀ unnormalised, m, l) to the workspace as a
//   16-byte aligned record of D + 4 floats.
// decode_reduce: merges the splits of each query head (the tutorial's
//   correction formula applied to every split against the common max):
//     M = max m_s,  L = Σ l_s 2^(m_s - M),  O = Σ O_s 2^(m_s - M) / L,
//     LSE = (M + log2 L) ln 2.
#include <atomic>

#include "fa_device.hpp"
#include "fa_kernels.h"

namespace fa {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <typename T> struct Mma16;
template <> struct Mma16<__bf16> {
  __device__ static __forceinline__ f32x4v mma(const bf16x8& a, const bf16x8& b, const f32x4v& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma16<_Float16> {
  __device__ static __forceinline__ f32x4v mma(const f16x8& a, const f16x8& b, const f32x4v& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <typename T, int D>
struct DecCfg {
  static constexpr int kWaves = 4;
  static constexpr int kPage = 16;                 // tokens per page
  static constexpr int kRowBytes = D * 2;
  static constexpr int kPageBytes = kPage * kRowBytes;
  static constexpr int kSlices = kPageBytes / 1024;  // 1 KiB wave loads per page
  static constexpr int kStageBytes = 2 * kPageBytes;  // V of two pages
  static constexpr int kKS = D / 32;               // 32-wide k blocks along d
  static constexpr int kDT = D / 16;               // 16-row M tiles of Oᵀ
  static constexpr int kPairOps = 2 * (kKS + kSlices);  // memory operations per page pair
  static_assert(kSlices >= 1 && kSlices * 1024 == kPageBytes, "page must split into 1 KiB loads");
};

struct SplitParams {
  const void* q;
  const void* kc;
  const void* vc;
  int B, Hq, Hkv, max_blocks, num_blocks, splits, n_qc;
  float c;
};

// The block table and sequence lengths are separate restrict-qualified
// arguments so that the compiler can prove them read-only and fetch them with
// scalar loads: a vector load would make the wave wait for every outstanding
// page load (they share one counter) and stall the pipeline each page.
template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_kernel(SplitParams p, const int* __restrict__ block_table,
                                                           const int* __restrict__ seq_lens,
                                                           float* __restrict__ part) {
  using C = DecCfg<T, D>;
  using TT = Tile<C::kRowBytes>;
  typedef typename Elem<T>::Frag Frag;

  // The two stages of every wave's V ring are separate LDS objects: the
  // compiler then sees that the pair being loaded never aliases the pair
  // being read, and lets the loads stay in flight across the reads.
  __shared__ __attribute__((aligned(1024))) char v_st0[C::kWaves * C::kStageBytes], v_st1[C::kWaves * C::kStageBytes];
  const int lane = lane_id(), w = wave_id();
  const int unit = blockIdx.x * C::kWaves + w;  // (split, query column tile) of this wave
  if (unit >= p.splits * p.n_qc) return;         // no barriers in this kernel
  const int split = unit / p.n_qc, qc = unit - split * p.n_qc;
  const int bhk = blockIdx.y;
  const int b = bhk / p.Hkv, hkv = bhk - b * p.Hkv;
  const int g = p.Hq / p.Hkv;
  lds_char* const ring0 = (lds_char*)v_st0 + w * C::kStageBytes;
  lds_char* const ring1 = (lds_char*)v_st1 + w * C::kStageBytes;

  const int i16 = lane & 15, G = lane >> 4;
  const int qi = qc * 16 + i16;                  // query head within the group (column)
  const bool q_ok = qi < g;
  const int hq = hkv * g + qi;

  // Tokens of the sequence, clamped to what its table row can address.
  const int seq_len = min(max(seq_lens[b], 0), p.max_blocks * C::kPage);
  const int n_pages = (seq_len + C::kPage - 1) / C::kPage;
  const int pg0 = (int)((int64_t)n_pages * split / p.splits);
  const int pg1 = (int)((int64_t)n_pages * (split + 1) / p.splits);
  const int tok_end = min(seq_len, pg1 * C::kPage);
  const int* table = block_table + (size_t)b * p.max_blocks;

  // Stage pages pg, pg+1: K into kr (lane: token row i16, d = 32ks + 8G ..
  // +7 of each page), V into ring buffer `st`.  Pages at or past pg1 get an
  // empty range, slots past the sequence end are clipped.
  typedef u32x4 KRegs[2][C::kKS];
  auto load_pair = [&](int pg, int st, KRegs& kr) __attribute__((always_inline)) {
    lds_char* sb = st ? ring1 : ring0;
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int page_idx = pg + u;
      uint32_t bytes = 0;
      size_t base = 0;
      if (page_idx < pg1) {
        const int page = table[page_idx];
        if (page >= 0 && page < p.num_blocks) {  // a bad table entry reads as a page of zeros
          base = ((size_t)page * p.Hkv + hkv) * C::kPageBytes;
          bytes = (uint32_t)min(C::kPage, seq_len - page_idx * C::kPage) * C::kRowBytes;
        }
      }
      const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.kc + base, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)p.vc + base, bytes);
#pragma unroll
      for (int ks = 0; ks < C::kKS; ks++) kr[u][ks] = buf_load16(rk, (uint32_t)i16 * C::kRowBytes + (4 * ks + G) * 16);
#pragma unroll
      for (int i = 0; i < C::kSlices; i++) {
        const int s = i * 64 + lane;
        const int row = s / TT::kChunks, pc = s % TT::kChunks;
        const uint32_t off = row * C::kRowBytes + ((pc ^ TT::key(row)) << 4);
        buf_load16_to_lds(rv, off, sb + u * C::kPageBytes + i * 1024);
      }
    }
  };

  const int n_pairs = (pg1 - pg0 + 1) / 2;
  KRegs ka, kb;  // K of the pair in stage 0 and in stage 1
  load_pair(pg0, 0, ka);

  // Qᵀ as the B operand: column = query head, k = d (8 per lane per 32-wide block).
  Frag qf[C::kKS];
  {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc((const char*)p.q + ((size_t)b * p.Hq + hkv * g) * C::kRowBytes, (uint32_t)g * C::kRowBytes);
    const uint32_t qoff = q_ok ? (uint32_t)qi * C::kRowBytes : 0xFFFFFFF0u;
#pragma unroll
    for (int ks = 0; ks < C::kKS; ks++)
      qf[ks] = __builtin_bit_cast(Frag, buf_load16(rq, qoff + (32 * ks + 8 * G) * 2));
  }

  f32x4v o[C::kDT];
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++) o[dt] = f32x4v{};
  float m = -INFINITY, l = 0.f;

  // One page pair: K from registers, V from ring stage st.
  auto pair = [&](int i, int st, const KRegs& kr) __attribute__((always_inline)) {
    const lds_char* vb = st ? ring1 : ring0;
    const int t0 = (pg0 + 2 * i) * C::kPage;  // first token of the pair

    // ---- Sᵀ for both pages: register r of page u holds token t0 + 16u + 4G + r.
    f32x4v s[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
      s[u] = f32x4v{};
#pragma unroll
      for (int ks = 0; ks < C::kKS; ks++) s[u] = Mma16<T>::mma(__builtin_bit_cast(Frag, kr[u][ks]), qf[ks], s[u]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float t = (t0 + 16 * u + 4 * G + r) < tok_end ? s[u][r] * p.c : -INFINITY;
        s[u][r] = t;
        mx = fmaxf(mx, t);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float pv[8], rs = 0.f;
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float e = fast_exp2(s[u][r] - m_use);
        pv[4 * u + r] = e;
        rs += e;
      }
    l = l * alpha + rs;
    m = m_new;
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int dt = 0; dt < C::kDT; dt++) o[dt] *= alpha;
    }
    const Frag pf = Elem<T>::pack(pv);  // slot t: token 4G + t of page 0 (t < 4), of page 1 (t >= 4)

    // ---- Oᵀ += Vᵀ Pᵀ.  Vᵀ slot t of lane (d = 16dt + i16, G) is V[token of slot t][d].
#pragma unroll
    for (int dt = 0; dt < C::kDT; dt++) {
      const int row = 4 * G + (i16 >> 2);
      const int col = 16 * dt + 4 * (lane & 3);
      const uint32_t off = TT::off(row, col >> 3) + ((col & 7) << 1);
      const i16x4 v0 = lds_read_tr16(vb, off);
      const i16x4 v1 = lds_read_tr16(vb + C::kPageBytes, off);
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 a8 = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      o[dt] = Mma16<T>::mma(__builtin_bit_cast(Frag, a8), pf, o[dt]);
    }
  };

  // Two pairs per trip so that both K register sets are compile-time objects.
  // Before a pair is used, only the newer pair's loads may still be in flight
  // (loads retire in issue order).  Loads and pairs past the split are issued
  // anyway: their pages have empty ranges and their tokens lie past tok_end,
  // so they add nothing, and no branch makes the waits conservative.
  for (int i = 0; i < n_pairs; i += 2) {
    load_pair(pg0 + 2 * (i + 1), 1, kb);
    wait_vmem_le<C::kPairOps>();
    pair(i, 0, ka);
    load_pair(pg0 + 2 * (i + 2), 0, ka);
    wait_vmem_le<C::kPairOps>();
    pair(i + 1, 1, kb);
  }
  wait_vmem();

  // ---- partial result: Oᵀ (unnormalised), m, l (summed over the 4 lane groups).
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (q_ok) {
    const size_t rec = (((size_t)b * p.Hq + hq) * p.splits + split) * (D + 4);
    float* dst = part + rec;
#pragma unroll
    for (int dt = 0; dt < C::kDT; dt++) {
      f32x4v v = o[dt];
      *(f32x4v*)(dst + 16 * dt + 4 * G) = v;  // d = 16dt + 4G + 0..3
    }
    if (G == 0) { dst[D] = m; dst[D + 1] = l; }
  }
}

// One wave per (sequence, query head), two memory round trips: lane s loads
// split s's max and sum (64 splits per round) while every lane loads its d
// values of all splits, then the wave reduces.  Splits are merged in a fixed
// order, so the result is deterministic.
template <typename T, int D, int SMAX>
__global__ __launch_bounds__(64) void decode_reduce_kernel(const float* __restrict__ part, T* __restrict__ out,
                                                           float* __restrict__ lse, int splits) {
  constexpr int kRec = D + 4;
  constexpr int kPer = (D + 63) / 64;
  const int bh = blockIdx.x, lane = threadIdx.x;
  const float* rec = part + (size_t)bh * splits * kRec;
  // Round trip 1 (issued together with round trip 2 below): split maxima and sums.
  float ms_l = -INFINITY, ls_l = 0.f;
  if (lane < splits) { ms_l = rec[(size_t)lane * kRec + D]; ls_l = rec[(size_t)lane * kRec + D + 1]; }
  float v[SMAX][kPer];
  if (splits <= SMAX) {
#pragma unroll
    for (int s = 0; s < SMAX; s++)
#pragma unroll
      for (int j = 0; j < kPer; j++) {
        const int d = lane + 64 * j;
        v[s][j] = (s < splits && d < D) ? rec[(size_t)s * kRec + d] : 0.f;
      }
  }
  float M = ms_l;
  for (int s = lane + 64; s < splits; s += 64) M = fmaxf(M, rec[(size_t)s * kRec + D]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float L = ms_l == -INFINITY ? 0.f : ls_l * fast_exp2(ms_l - M);
  for (int s = lane + 64; s < splits; s += 64) {
    const float ms = rec[(size_t)s * kRec + D];
    if (ms != -INFINITY) L = fmaf(rec[(size_t)s * kRec + D + 1], fast_exp2(ms - M), L);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off, 64);
  // Weight of split s: 2^(m_s - M), 0 for splits that saw no key.
  const float wl = ms_l == -INFINITY ? 0.f : fast_exp2(ms_l - M);
  float acc[kPer];
#pragma unroll
  for (int j = 0; j < kPer; j++) acc[j] = 0.f;
  if (splits <= SMAX) {
#pragma unroll
    for (int s = 0; s < SMAX; s++) {
      const float wgt = __shfl(wl, s, 64);
#pragma unroll
      for (int j = 0; j < kPer; j++) acc[j] = fmaf(v[s][j], wgt, acc[j]);
    }
  } else {
    for (int s = 0; s < splits; s++) {
      const float* r = rec + (size_t)s * kRec;
      const float ms = r[D];
      const float wgt = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
#pragma unroll
      for (int j = 0; j < kPer; j++) {
        const int d = lane + 64 * j;
        if (d < D) acc[j] = fmaf(r[d], wgt, acc[j]);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int d = lane + 64 * j;
    if (d < D) out[(size_t)bh * D + d] = (T)(acc[j] * inv);
  }
  if (lse != nullptr && lane == 0) lse[bh] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
}

template <typename T, int D>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  using C = DecCfg<T, D>;
  SplitParams p;
  p.q = a.q; p.kc = a.k_cache; p.vc = a.v_cache; p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.max_blocks = a.max_blocks; p.num_blocks = a.num_blocks;
  p.splits = a.splits;
  const int g = a.Hq / a.Hkv;
  p.n_qc = (g + 15) / 16;
  p.c = a.scale * kLog2e;
  const int units = a.splits * p.n_qc;
  dim3 grid((units + C::kWaves - 1) / C::kWaves, a.B * a.Hkv);
  hipLaunchKernelGGL((decode_split_kernel<T, D>), grid, dim3(64 * C::kWaves), 0, stream, p, a.block_table,
                     a.seq_lens, a.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Up to 32 splits are merged from registers loaded in one round trip.
  if (a.splits <= 16)
    hipLaunchKernelGGL((decode_reduce_kernel<T, D, 16>), dim3(a.B * a.Hq), dim3(64), 0, stream, a.part, (T*)a.o,
                       a.lse, a.splits);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<T, D, 32>), dim3(a.B * a.Hq), dim3(64), 0, stream, a.part, (T*)a.o,
                       a.lse, a.splits);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const DecodeArgs& a, hipStream_t s) {
  switch (a.d) {
    case 32: return launch_typed<T, 32>(a, s);
    case 64: return launch_typed<T, 64>(a, s);
    case 128: return launch_typed<T, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

// Scratch area of the allocation-free decode entry point: the split records
// ([B, Hq, splits, d + 4] float32) of one call.  Every GPU the library runs on
// holds its own copy until the process ends.  Host code never uses the
// array's name as an address: decode_scratch_area() resolves the device copy
// with hipGetSymbolAddress once per device and passes that pointer on.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];

}  // namespace

hipError_t decode_scratch_area(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    // With this device current: the address of this device's copy.  Racing
    // first calls store the same value.
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 1: return launch_dtype<_Float16>(a, stream);
    case 2: return launch_dtype<__bf16>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
