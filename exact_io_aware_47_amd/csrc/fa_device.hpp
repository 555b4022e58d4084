// fa_device.hpp -- gfx950 device building blocks shared by the attention kernels.
//
// Matrix-core fragments (CDNA4 MFMA, wave64), bounds-checked buffer loads
// (direct to LDS or to registers), the swizzled LDS tile addressing, the
// transposing LDS read, and the float32 <-> 16-bit conversions.
//
// MFMA layouts used throughout (v_mfma_f32_32x32x16_{bf16,f16} and the
// float32 v_mfma_f32_32x32x2f32), with lane l and half h = l / 32:
//   A (32 x 16, M x K): lane l holds row l % 32, k = 8h .. 8h+7
//   B (16 x 32, K x N): lane l holds column l % 32, k = 8h .. 8h+7
//   C (32 x 32)       : lane l, register r holds column l % 32 and
//                       row 8*(r/4) + 4h + (r%4)
// For float32 a 16-wide k block is eight 32x32x2 products; product t takes
// slot t of each half, so lane half h still supplies k = 8h + t.  Which k a
// slot stands for never matters for a contraction as long as A and B agree.
//
// Row permutation sigma: if the A rows fed to an MFMA are permuted by sigma
// (swap bits 2 and 3 of the row index), the C register r of lane half h holds
// row 16*(r/8) + 8h + (r%8).  Registers 0..7 (and 8..15) then form exactly the
// B-operand layout of a following product that contracts over those rows, so
// P = softmax(S) can feed the next MFMA straight from registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Reinterpret a 32-bit word as float.  Takes the word by value: bit-casting a
// vector element expression in place (v[i]) reads element 0 with this
// compiler, so element accesses always go through this function.
__device__ __forceinline__ float as_float(uint32_t x) { return __builtin_bit_cast(float, x); }

// Compile-time integer as a value (selects unrolled variants in lambdas).
template <int N> struct Int { static constexpr int value = N; };

// fn(Int<B>{}), fn(Int<B + 1>{}), ..., fn(Int<E - 1>{}).
template <int B, int E, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (B < E) {
    fn(Int<B>{});
    static_for<B + 1, E>(fn);
  }
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / 64); }

// --------------------------------------------------------------------------
// Element types.  Frag<T>: one lane's 8 consecutive k values of an A or B
// operand for a 16-wide k block.
// --------------------------------------------------------------------------
template <typename T> struct Elem;

template <> struct Elem<__bf16> {
  typedef bf16x8 Frag;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ f32x16 mma(const Frag& a, const Frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ Frag pack(const float* x) {
    Frag f;
#pragma unroll
    for (int i = 0; i < 8; i++) f[i] = (__bf16)x[i];  // v_cvt_pk_bf16_f32, round to nearest even
    return f;
  }
  __device__ static __forceinline__ float to_f32(__bf16 x) { return (float)x; }
  __device__ static __forceinline__ Frag negate(const Frag& f) {  // flip the sign bits (exact)
    return __builtin_bit_cast(Frag, __builtin_bit_cast(u32x4, f) ^ 0x80008000u);
  }
};

template <> struct Elem<_Float16> {
  typedef f16x8 Frag;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ f32x16 mma(const Frag& a, const Frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ Frag pack(const float* x) {
    Frag f;
#pragma unroll
    for (int i = 0; i < 8; i++) f[i] = (_Float16)x[i];  // round to nearest even
    return f;
  }
  __device__ static __forceinline__ float to_f32(_Float16 x) { return (float)x; }
  __device__ static __forceinline__ Frag negate(const Frag& f) {
    return __builtin_bit_cast(Frag, __builtin_bit_cast(u32x4, f) ^ 0x80008000u);
  }
};

struct F32Frag { float v[8]; };

template <> struct Elem<float> {
  typedef F32Frag Frag;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ f32x16 mma(const Frag& a, const Frag& b, f32x16 c) {
#pragma unroll
    for (int t = 0; t < 8; t++) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[t], b.v[t], c, 0, 0, 0);
    return c;
  }
  __device__ static __forceinline__ Frag pack(const float* x) {
    Frag f;
#pragma unroll
    for (int i = 0; i < 8; i++) f.v[i] = x[i];
    return f;
  }
  __device__ static __forceinline__ float to_f32(float x) { return x; }
  __device__ static __forceinline__ Frag negate(Frag f) {
#pragma unroll
    for (int i = 0; i < 8; i++) f.v[i] = -f.v[i];
    return f;
  }
};

// --------------------------------------------------------------------------
// Buffer resources: raw (stride 0) descriptors whose byte range is checked by
// the hardware.  Loads beyond num_bytes return zero, stores beyond it are
// dropped, so ragged tails need no per-lane branches.
// --------------------------------------------------------------------------
constexpr int kBufferFlags = 0x00020000;  // gfx9 word 3: 32-bit data format, raw addressing

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, kBufferFlags);
}

// --------------------------------------------------------------------------
// Sequences of a batch.  Head h of sequence b is one contiguous [n, d] slab
// that starts at row H * t + h * n of its tensor, where t is the sequence's
// first token and n its length (H = Hq for Q/O/dO/dQ/LSE, Hkv for K/V/dK/dV).
// A dense batch has t = b * N and n = N; a packed batch (cu_q != nullptr)
// takes t and n from the cumulative lengths cu_q / cu_k ([B + 1] int32), and
// N then bounds every length.  A sequence whose bounds are not
// 0 <= cu[b] <= cu[b + 1] <= total with a length <= N is read as empty, so a
// malformed array can never send a slab outside its tensor.
// --------------------------------------------------------------------------
struct SeqRows {
  int nq, nk;  // query and key counts of the sequence
  int tq, tk;  // first query and first key token of the sequence
};

__device__ __forceinline__ SeqRows seq_rows(const int* cu_q, const int* cu_k, int b, int Nq, int Nk, int tot_q,
                                            int tot_k) {
  if (cu_q == nullptr) return SeqRows{Nq, Nk, b * Nq, b * Nk};
  const int a0 = cu_q[b], a1 = cu_q[b + 1], c0 = cu_k[b], c1 = cu_k[b + 1];
  const bool ok = 0 <= a0 && a0 <= a1 && a1 <= tot_q && a1 - a0 <= Nq && 0 <= c0 && c0 <= c1 && c1 <= tot_k &&
                  c1 - c0 <= Nk;
  return ok ? SeqRows{a1 - a0, c1 - c0, a0, c0} : SeqRows{0, 0, 0, 0};
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS: lane L of the wave
// writes lds_wave_base + 16 * L (lds_wave_base must be wave-uniform).
__device__ __forceinline__ void buf_load16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, lds_char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, off, 0, 0, 0);
}

// s_waitcnt through the compiler intrinsic (not inline asm), so that the
// compiler's own wait insertion sees which loads have already been drained.
// gfx9 encoding: vmcnt = bits [3:0] and [15:14], expcnt = [6:4], lgkmcnt = [11:8].
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vmem() { wait_vmem_le<0>(); }
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Work-group barrier that lets buffer-to-LDS loads stay in flight: only this
// wave's LDS accesses are drained before s_barrier, and the "memory" clobber
// keeps the compiler from moving memory accesses across it.  Code that needs
// staged tiles to be visible calls wait_vmem() first.
__device__ __forceinline__ void barrier_lds() {
  wait_lds();
  asm volatile("s_barrier" ::: "memory");
}

// --------------------------------------------------------------------------
// LDS tiles: rows of ROW_BYTES stored as 16-byte chunks whose position in a
// row is XOR-permuted by a per-row key.  The key is chosen so that both read
// patterns of the kernels hit distinct banks (64 banks x 4 B = 256 B):
//   row fragments   : 16 consecutive rows at one chunk column land in 16
//                     distinct 16-byte bank groups;
//   column fragments: 4 consecutive rows at an aligned group of 4 chunk
//                     columns (a transposing read) land in 4 distinct
//                     64-byte bank segments.
// With 16+ chunks per row the key 4*(row%4) + (row/4)%4 is a bijection on 16
// rows and spreads any 4 consecutive rows over the 4 segments; with 8 chunks
// (two rows per 256 B) bit 2 of the key is bit 1 of the row; with 4 chunks
// (four rows per 256 B) the row itself picks the segment.
// --------------------------------------------------------------------------
template <int ROW_BYTES>
struct Tile {
  static constexpr int kChunks = ROW_BYTES / 16;  // chunks per row
  static_assert(kChunks == 4 || kChunks == 8 || kChunks % 16 == 0, "unsupported row size");
  __device__ static __forceinline__ int key(int row) {
    if constexpr (kChunks >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else if constexpr (kChunks == 8) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    else return (row >> 2) & 3;
  }
  // byte offset of logical chunk c of row `row`
  __device__ static __forceinline__ uint32_t off(int row, int c) {
    return (uint32_t)(row * ROW_BYTES + ((c ^ key(row)) << 4));
  }
};

// Stage ROWS rows of ROW_BYTES, starting at byte g0 of resource r, into a
// swizzled LDS tile.  The tile splits into 1 KiB slices of 64 lanes x 16 B;
// each of the WAVES waves moves an equal share.  Physical slot s holds logical
// chunk (s % chunks) ^ key(row) of row s / chunks; rows past the resource's
// range read as zero.
// PAGED: the tile's rows come from 16-row pages.  The rows one wave moves
// always lie in a single page (see dma_wave_row0), so r is that wave's page
// (its first row at byte 0) and tile row i sits at in-page row i % 16.
template <int ROW_BYTES, int ROWS, int WAVES>
struct DmaShape {
  static constexpr int kSlices = ROWS * ROW_BYTES / 1024;
  // With fewer slices than waves, the first kSlices waves move one each.
  static constexpr int kPer = kSlices >= WAVES ? kSlices / WAVES : 1;
  static constexpr int kActive = kSlices >= WAVES ? WAVES : kSlices;
  static constexpr int kWaveRows = kPer * 1024 / ROW_BYTES;  // rows moved by one wave
  static_assert(kSlices * 1024 == ROWS * ROW_BYTES && kPer * kActive == kSlices, "tile must split into whole wave slices");
};

// First tile row moved by wave w (waves at or past kActive move nothing).
template <int ROW_BYTES, int ROWS, int WAVES>
__device__ __forceinline__ int dma_wave_row0(int w) {
  return w * DmaShape<ROW_BYTES, ROWS, WAVES>::kWaveRows;
}

template <int ROW_BYTES, int ROWS, int WAVES, bool PAGED = false>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t r, uint32_t g0, lds_char* tile, int w, int lane) {
  using TT = Tile<ROW_BYTES>;
  using S = DmaShape<ROW_BYTES, ROWS, WAVES>;
  static_assert(!PAGED || (S::kWaveRows <= 16 && 16 % S::kWaveRows == 0 && ROWS % 16 == 0),
                "a wave's rows must stay within one 16-row page");
  if (S::kActive < WAVES && w >= S::kActive) return;
#pragma unroll
  for (int i = 0; i < S::kPer; i++) {
    const int s0 = (w * S::kPer + i) * 64;
    const int s = s0 + lane;
    const int row = s / TT::kChunks, pc = s % TT::kChunks;
    buf_load16_to_lds(r, g0 + (PAGED ? (row & 15) : row) * ROW_BYTES + ((pc ^ TT::key(row)) << 4), tile + s0 * 16);
  }
}

__device__ __forceinline__ u32x4 lds_read16(const lds_char* base, uint32_t off) {
  return *(const __attribute__((address_space(3))) u32x4*)(base + off);
}
__device__ __forceinline__ float lds_read_f32(const lds_char* base, uint32_t off) {
  return *(const __attribute__((address_space(3))) float*)(base + off);
}
// Transposing read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane
// j supplies the address of 4 consecutive 16-bit elements (row j/4 of a 4-row
// block, columns 4*(j%4)..+3); lane i receives column i of that 4 x 16 block,
// i.e. the 4 elements (row 0..3, column i).
__device__ __forceinline__ i16x4 lds_read_tr16(const lds_char* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(base + off));
}

// sigma: swap bits 2 and 3 of a row index within a 32-row MFMA tile.
__device__ __forceinline__ int sigma(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// --------------------------------------------------------------------------
// Instruction schedule of a block of LDS fragment reads feeding MFMAs: the
// first PD MFMAs' reads are issued up front, then every MFMA is followed by
// the reads of the MFMA PD places later, so each read has PD MFMA slots
// (32 cycles each) to return.  NR reads, NM MFMAs, NR a multiple of NM.
// --------------------------------------------------------------------------
template <int NR, int NM, int PD>
__device__ __forceinline__ void sched_reads_ahead() {
  static_assert(NR % NM == 0, "reads per MFMA must be whole");
  constexpr int kMaskMfma = 0x008, kMaskDsRead = 0x100;
  constexpr int r = NR / NM;
  constexpr int pd = PD < NM ? PD : NM;  // short blocks: all reads up front
  __builtin_amdgcn_sched_group_barrier(kMaskDsRead, pd * r, 0);
#pragma unroll
  for (int i = 0; i < NM - pd; i++) {
    __builtin_amdgcn_sched_group_barrier(kMaskMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kMaskDsRead, r, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMaskMfma, pd, 0);
}

// --------------------------------------------------------------------------
// Cross-lane helpers
// --------------------------------------------------------------------------
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// The larger of a and b as IEEE maximum (NaN if either is NaN).  On gfx950
// this is v_maximum3_f32 on the operands as they are; fmaxf (maxnum) first
// quiets every operand that might be a signalling NaN with one more max.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max(x, x of the lane 32 places away) in every lane, on the VALU
// (v_permlane32_swap exchanges the upper half of one operand with the lower
// half of the other; with both operands x the two results hold x's lower and
// upper halves in both halves).
__device__ __forceinline__ float max_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return vmax(as_float((uint32_t)r[0]), as_float((uint32_t)r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return as_float((uint32_t)r[0]) + as_float((uint32_t)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// --------------------------------------------------------------------------
// Operand fragments
// --------------------------------------------------------------------------
template <typename T>
struct Frags {
  typedef typename Elem<T>::Frag Frag;
  static constexpr int kES = Elem<T>::kBytes;

  // Row fragment from a swizzled LDS tile: elements 16*ks + 8h .. +7 of `row`
  // (A operand with rows = tile rows, k = tile columns).
  template <typename TileT>
  __device__ static __forceinline__ Frag lds_row(const lds_char* base, int row, int ks, int h) {
    if constexpr (kES == 2) {
      return __builtin_bit_cast(Frag, lds_read16(base, TileT::off(row, 2 * ks + h)));
    } else {
      u32x4 a = lds_read16(base, TileT::off(row, 4 * ks + 2 * h));
      u32x4 b = lds_read16(base, TileT::off(row, 4 * ks + 2 * h + 1));
      Frag f;
#pragma unroll
      for (int i = 0; i < 4; i++) { f.v[i] = as_float(a[i]); f.v[4 + i] = as_float(b[i]); }
      return f;
    }
  }

  // Column fragment from a swizzled LDS tile: rows r0 + 8h + t (t = 0..7) of
  // column c0 + (lane % 32)  (A operand of the transposed tile: rows = tile
  // columns, k = tile rows).  16-bit types use two transposing reads.
  template <typename TileT>
  __device__ static __forceinline__ Frag lds_col(const lds_char* base, int r0, int c0, int lane) {
    const int h = lane >> 5;
    if constexpr (kES == 2) {
      const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      i16x4 t[2];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int row = r0 + 8 * h + 4 * u + ((lane & 15) >> 2);
        t[u] = lds_read_tr16(base, TileT::off(row, col >> 3) + ((col & 7) << 1));
      }
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      i16x8 c = {t[0][0], t[0][1], t[0][2], t[0][3], t[1][0], t[1][1], t[1][2], t[1][3]};
      return __builtin_bit_cast(Frag, c);
    } else {
      const int col = c0 + (lane & 31);
      Frag f;
#pragma unroll
      for (int t = 0; t < 8; t++) {
        const int row = r0 + 8 * h + t;
        f.v[t] = lds_read_f32(base, TileT::off(row, col >> 2) + ((col & 3) << 2));
      }
      return f;
    }
  }

  // Row fragment straight from a global [rows][D] slab (bounds-checked: rows
  // past the resource's range read as zero).
  template <int D>
  __device__ static __forceinline__ Frag global_row(__amdgpu_buffer_rsrc_t r, int row, int ks, int h) {
    const uint32_t off = (uint32_t)row * (D * kES) + (uint32_t)(16 * ks + 8 * h) * kES;
    if constexpr (kES == 2) {
      return __builtin_bit_cast(Frag, buf_load16(r, off));
    } else {
      u32x4 a = buf_load16(r, off), b = buf_load16(r, off + 16);
      Frag f;
#pragma unroll
      for (int i = 0; i < 4; i++) { f.v[i] = as_float(a[i]); f.v[4 + i] = as_float(b[i]); }
      return f;
    }
  }

  // The same fragments from precomputed per-lane byte offsets (16-bit types):
  // a row fragment is one 16-byte read, a column fragment two transposing reads.
  __device__ static __forceinline__ Frag lds_row_at(const lds_char* base, uint32_t off) {
    static_assert(kES == 2, "16-bit types only");
    return __builtin_bit_cast(Frag, lds_read16(base, off));
  }
  __device__ static __forceinline__ Frag lds_col_at(const lds_char* base, uint32_t off0, uint32_t off1) {
    static_assert(kES == 2, "16-bit types only");
    const i16x4 a = lds_read_tr16(base, off0), b = lds_read_tr16(base, off1);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(Frag, c);
  }
  // Offsets used by lds_row(base, row, ks, h) and lds_col(base, r0 = 0, c0, lane)
  // for a tile of TileT rows; adding 32*mt or 16*ps rows only adds a constant.
  template <typename TileT>
  __device__ static __forceinline__ uint32_t row_off(int row, int ks, int h) {
    return TileT::off(row, 2 * ks + h);
  }
  template <typename TileT>
  __device__ static __forceinline__ uint32_t col_off(int c0, int u, int lane) {
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int row = 8 * (lane >> 5) + 4 * u + ((lane & 15) >> 2);
    return TileT::off(row, col >> 3) + ((col & 7) << 1);
  }

  // Store 4 consecutive elements (rounded to T) at byte offset `off`.
  __device__ static __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t off, float a, float b, float c, float d) {
    if constexpr (kES == 2) {
      typedef T t2 __attribute__((ext_vector_type(2)));
      t2 x = {(T)a, (T)b}, y = {(T)c, (T)d};
      u32x2 w = {__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y)};
      buf_store8(r, off, w);
    } else {
      u32x4 w = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                 __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
      buf_store16(r, off, w);
    }
  }
};

}  // namespace fa
