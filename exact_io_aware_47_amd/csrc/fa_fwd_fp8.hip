// fa_fwd_fp8.hip -- attention forward on FP8 (E4M3) inputs for gfx950.
//
// Same method as the 16-bit forward (tutorial "FlashAttention and efficient
// attention kernels": "Online softmax", "Correction formula", "Forward";
// concept page "Flash-Attention", "Core idea"), with the FP8 route the
// concept page names among FlashAttention-3's techniques ("Key
// observations"): Q, K, V arrive as E4M3 codes with one float32 descale per
// tensor, both products run on the FP8 matrix cores, and the probabilities
// are rounded to E4M3 before the second product.
//
// Products: v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales (C 32x32
// float32 += A 32x64 * B 64x32).  Which of the 64 k indices a lane's 32 byte
// slots stand for is never needed: A and B take the same slots, so any
// assignment that is the same on both sides contracts correctly.
//   Sᵀ = K Qᵀ : A rows are keys, read in the order pi below, B columns are
//               queries (Q rows kept in registers), k = d.
//   Oᵀ = Vᵀ Pᵀ: A rows are d, k = keys; B = Pᵀ straight from the score
//               registers.  With the pi row order, lane half h of a query
//               column holds the tile's keys 32h .. 32h+31 in its 32 score
//               registers (two 32-key M tiles x 16), which become the 32
//               bytes of its B operand in key order, so the A operand is 32
//               consecutive keys of one row of Vᵀ.
// V is staged transposed: a pre-pass writes Vᵀ per 64-key tile ([d][64]
// bytes, keys past Nk zero) into the workspace, so that a Vᵀ tile is one
// contiguous block that the tile loader moves like any other.
//
// Softmax: as in the 16-bit kernel (log2 domain, one max exchange between
// the lane halves per tile), with the running max moved only when it grows
// by more than 2^2, and P taken as exp2(s*c - m + 6): every P then lies in
// (0, 2^8], inside E4M3's range (448), and values down to 2^-15 of the max
// stay representable.  The row sum l adds the same (unrounded) values, so
// the factor 2^6 cancels in O = Oᵀ / l; LSE removes it explicitly.
#include "fa_device.hpp"
#include "fa_kernels.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// C += A B on E4M3 operands (format code 0 for A and B; E8M0 block scale
// 127 = 2^0 for both).
__device__ __forceinline__ f32x16 mma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 32 bytes = two 16-byte chunks of a swizzled LDS tile.
__device__ __forceinline__ i32x8 lds_read32(const lds_char* base, uint32_t off0, uint32_t off1) {
  const u32x4 a = lds_read16(base, off0), b = lds_read16(base, off1);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

constexpr int kVtKeys = 64;  // keys per staged Vᵀ tile

// ---------------------------------------------------------------------------
// Pre-pass: Vt[b][hkv][tile][d][64] = V[b][hkv][64 * tile + key][d], zero past Nk.
// Each thread moves a 4-key x 16-d block: four 16-byte row loads, four 4x4
// byte transposes in registers (v_perm_b32), sixteen 4-byte stores.  Sixteen
// consecutive threads cover the 64 keys of a tile, so every output row of Vᵀ
// is written as one contiguous 64-byte run.
// ---------------------------------------------------------------------------
// Bytes j of a, b, c, d (j = 0..3) as one word, for each j: the transpose of a
// 4x4 byte block held as four row words.
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t* o) {
  // perm(x, y, sel): byte i of the result is byte sel_i of {x:y} (y = bytes 0-3, x = bytes 4-7).
  const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);  // c2 d2 c3 d3
  o[0] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);  // a0 b0 c0 d0
  o[1] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);  // a1 b1 c1 d1
  o[2] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);  // a2 b2 c2 d2
  o[3] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);  // a3 b3 c3 d3
}

template <int D>
__global__ __launch_bounds__(256) void fp8_vt_kernel(const uint8_t* __restrict__ v, uint8_t* __restrict__ vt,
                                                     int Nk, int n_tiles) {
  constexpr int kBlocks = (kVtKeys / 4) * (D / 16);  // 4 x 16 blocks per tile
  const int tile = blockIdx.x;
  const size_t bh = blockIdx.y;
  const __amdgpu_buffer_rsrc_t src = make_rsrc(v + bh * (size_t)Nk * D, (uint32_t)Nk * D);
  uint8_t* dst = vt + (bh * n_tiles + tile) * (size_t)(D * kVtKeys);
  for (int t = threadIdx.x; t < kBlocks; t += 256) {
    const int kg = t % (kVtKeys / 4), dg = t / (kVtKeys / 4);
    const int key0 = tile * kVtKeys + 4 * kg, d0 = 16 * dg;
    u32x4 r[4];  // rows key0 .. key0+3, bytes d0 .. d0+15 (zero past Nk)
#pragma unroll
    for (int i = 0; i < 4; i++) r[i] = buf_load16(src, (uint32_t)(key0 + i) * D + d0);
#pragma unroll
    for (int c = 0; c < 4; c++) {
      uint32_t o[4];
      transpose4x4(r[0][c], r[1][c], r[2][c], r[3][c], o);
#pragma unroll
      for (int j = 0; j < 4; j++) *(uint32_t*)(dst + (size_t)(d0 + 4 * c + j) * kVtKeys + 4 * kg) = o[j];
    }
  }
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
// Work-groups of 4 waves (128 query rows, 32 per wave): at head size 128 a
// wave takes 156 registers, so three work-groups share a compute unit (three
// waves per SIMD, each from its own work-group and out of step with the
// others); an 8-wave work-group puts two waves on each SIMD and leaves no
// room for a second one.
template <int D>
struct Fp8Cfg {
  static constexpr int kWaves = 4;
  static constexpr int kBR = 32 * kWaves;  // query rows per work-group
  static constexpr int kBC = kVtKeys;      // keys per tile
  static constexpr int kKB = D / 64;       // 64-wide k blocks of Sᵀ along d
  static constexpr int kDT = D / 32;       // 32-row M tiles of Oᵀ
  static constexpr int kTileBytes = kBC * D;  // a K tile (64 x D) and a Vᵀ tile (D x 64)
};

struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* vt;  // staged Vᵀ tiles [B, Hkv, n_ktiles, D, 64]
  void* o;            // bf16 [B, Hq, Nq, D]
  float* lse;
  int B, Hq, Hkv, Nq, Nk, n_ktiles;
  float c;          // |scale * q_descale * k_descale| * log2(e), or 2^-100 for zero
  int neg_q;        // that product is negative: Q's sign bits are flipped instead
  float v_descale;
};

constexpr float kTauFp8 = 2.0f;   // running-max threshold (log2 units)
constexpr float kPShift = 6.0f;   // P = exp2(s*c - m + kPShift) <= 2^(kTauFp8 + kPShift) = 256

// Key of A row i of M tile mt in Sᵀ: lane half h of the result then holds
// keys 32h + 16mt + r in its registers r = 0..15.
__device__ __forceinline__ int pi_row(int i, int mt) {
  return 32 * ((i >> 2) & 1) + 16 * mt + 4 * (i >> 3) + (i & 3);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_fp8_kernel(Fp8Params p) {
  using C = Fp8Cfg<D>;
  using TK = Tile<D>;        // K tile: 64 rows of D bytes
  using TV = Tile<C::kBC>;   // Vᵀ tile: D rows of 64 bytes
  __shared__ __attribute__((aligned(1024))) char k_lds0[C::kTileBytes], k_lds1[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[C::kTileBytes], v_lds1[C::kTileBytes];

  // Block -> (query tile, batch, head); heavy causal tiles first.
  const int bh_count = p.B * p.Hq;
  const int id = blockIdx.x;
  const int bh = id % bh_count;
  const int n_qt = (p.Nq + C::kBR - 1) / C::kBR;
  const int qt = CAUSAL ? (n_qt - 1 - id / bh_count) : id / bh_count;
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);

  const int lane = lane_id(), w = wave_id();
  const int h = lane >> 5, col = lane & 31;
  const int q0 = qt * C::kBR;
  const int qw = q0 + 32 * w;
  const int qrow = qw + col;
  const int diag = p.Nk - p.Nq;

  const size_t q_slab = (size_t)bh * p.Nq * D;
  const size_t kv_bh = (size_t)b * p.Hkv + hkv;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + q_slab, (uint32_t)p.Nq * D);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + kv_bh * p.Nk * D, (uint32_t)p.Nk * D);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(p.vt + kv_bh * p.n_ktiles * C::kTileBytes, (uint32_t)p.n_ktiles * C::kTileBytes);

  int n_tiles = p.n_ktiles;
  if (CAUSAL) {
    const int last_key = min(q0 + C::kBR, p.Nq) - 1 + diag;
    n_tiles = last_key < 0 ? 0 : min(n_tiles, last_key / C::kBC + 1);
  }
  auto load_tile = [&](int j, lds_char* kd, lds_char* vd) __attribute__((always_inline)) {
    dma_tile<D, C::kBC, C::kWaves>(rk, (uint32_t)j * C::kTileBytes, kd, w, lane);
    dma_tile<C::kBC, D, C::kWaves>(rv, (uint32_t)j * C::kTileBytes, vd, w, lane);
  };
  if (n_tiles > 0) load_tile(0, (lds_char*)k_lds0, (lds_char*)v_lds0);

  // Qᵀ as the B operand: lane holds row qrow, bytes 64 kb + 32 h .. +31.
  i32x8 qf[C::kKB];
#pragma unroll
  for (int kb = 0; kb < C::kKB; kb++) {
    const uint32_t off = (uint32_t)qrow * D + 64 * kb + 32 * h;
    const u32x4 a = buf_load16(rq, off), bq = buf_load16(rq, off + 16);
    qf[kb] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)bq[0], (int)bq[1], (int)bq[2], (int)bq[3]};
  }
  // c > 0, so the max of c*s is c*max(s); a negative scale flips Q's sign
  // bits instead (exact).
  if (p.neg_q) {
#pragma unroll
    for (int kb = 0; kb < C::kKB; kb++) qf[kb] ^= (int)0x80808080;
  }
  const float c = p.c;

  // Per-lane LDS offsets of the A fragments.
  uint32_t koff[2][C::kKB][2], voff[C::kDT][2];
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int kb = 0; kb < C::kKB; kb++)
#pragma unroll
      for (int u = 0; u < 2; u++) koff[mt][kb][u] = TK::off(pi_row(col, mt), 4 * kb + 2 * h + u);
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++)
#pragma unroll
    for (int u = 0; u < 2; u++) voff[dt][u] = TV::off(32 * dt + col, 2 * h + u);

  f32x16 o[C::kDT];
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++) o[dt] = f32x16{};
  float m = -INFINITY;  // running (possibly stale) max of c*s, log2 domain
  float l = 0.f;        // this lane's share of the running sum

  auto active = [&](int j) __attribute__((always_inline)) {
    return !CAUSAL || j * C::kBC <= qw + 31 + diag;
  };

  auto tile = [&](int j, const lds_char* kb_, const lds_char* vb_) __attribute__((always_inline)) {
    // ---- Sᵀ = K Qᵀ; register r of M tile mt holds key k0 + 32h + 16mt + r.
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kb = 0; kb < C::kKB; kb++)
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
        s[mt] = mma_fp8(lds_read32(kb_, koff[mt][kb][0], koff[mt][kb][1]), qf[kb], s[mt]);
    const int k0 = j * C::kBC;
    if ((k0 + C::kBC > p.Nk) || (CAUSAL && k0 + C::kBC - 1 > qw + diag)) {
      const int horizon = CAUSAL ? min(qrow + diag, p.Nk - 1) : p.Nk - 1;
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int r = 0; r < 16; r++)
          if (k0 + 32 * h + 16 * mt + r > horizon) s[mt][r] = -INFINITY;
    }
    float x[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int r = (mt == 0 ? 4 : 0); r < 16; r += 4)
#pragma unroll
        for (int i = 0; i < 4; i++) x[i] = vmax(x[i], s[mt][r + i]);
    const float mx = max_halves(vmax(vmax(x[0], x[1]), vmax(x[2], x[3]))) * c;
    const bool grow = mx > m + kTauFp8;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m - mx) : 1.f;
      m = grow ? mx : m;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::kDT; dt++) o[dt] *= alpha;
    }
    const float m_use = (m == -INFINITY ? 0.f : m) - kPShift;
    float rs[4];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        s[mt][r] = fast_exp2(fmaf(s[mt][r], c, -m_use));
        rs[r & 3] = (mt == 0 && r < 4) ? s[mt][r] : rs[r & 3] + s[mt][r];
      }
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    // ---- Pᵀ as E4M3 bytes in key order (byte t = key 32h + t).
    i32x8 pf;
#pragma unroll
    for (int wd = 0; wd < 8; wd++) {
      const int mt = wd >> 2, r = 4 * (wd & 3);
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(s[mt][r], s[mt][r + 1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(s[mt][r + 2], s[mt][r + 3], v, true);
      pf[wd] = v;
    }
    // ---- Oᵀ += Vᵀ Pᵀ.
#pragma unroll
    for (int dt = 0; dt < C::kDT; dt++) o[dt] = mma_fp8(lds_read32(vb_, voff[dt][0], voff[dt][1]), pf, o[dt]);
  };

  wait_vmem();
  barrier_lds();
  // Two tiles per trip so that every LDS buffer is a compile-time object.
  for (int j = 0; j < n_tiles; j += 2) {
    if (j + 1 < n_tiles) load_tile(j + 1, (lds_char*)k_lds1, (lds_char*)v_lds1);
    if (active(j)) tile(j, (const lds_char*)k_lds0, (const lds_char*)v_lds0);
    wait_vmem();
    barrier_lds();
    if (j + 1 < n_tiles) {
      if (j + 2 < n_tiles) load_tile(j + 2, (lds_char*)k_lds0, (lds_char*)v_lds0);
      if (active(j + 1)) tile(j + 1, (const lds_char*)k_lds1, (const lds_char*)v_lds1);
      wait_vmem();
      barrier_lds();
    }
  }

  // ---- epilogue: O = v_descale * Oᵀ / l in bf16, LSE = (m + log2 l - shift) ln 2.
  const float lt = sum_halves(l);
  const float inv = lt > 0.f ? p.v_descale / lt : 0.f;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc((char*)p.o + q_slab * 2, (uint32_t)p.Nq * D * 2);
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++)
#pragma unroll
    for (int a4 = 0; a4 < 4; a4++) {
      const int d0 = 32 * dt + 8 * a4 + 4 * h;
      Frags<__bf16>::store4(ro, (uint32_t)qrow * D * 2 + d0 * 2, o[dt][4 * a4] * inv, o[dt][4 * a4 + 1] * inv,
                            o[dt][4 * a4 + 2] * inv, o[dt][4 * a4 + 3] * inv);
    }
  if (h == 0) {
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + (size_t)bh * p.Nq, (uint32_t)p.Nq * 4);
    const float lse = lt > 0.f ? (m + fast_log2(lt) - kPShift) * kLn2 : -INFINITY;
    buf_store4(rl, (uint32_t)qrow * 4, __builtin_bit_cast(uint32_t, lse));
  }
}

template <int D, bool CAUSAL>
hipError_t launch_typed(const Fp8FwdArgs& a, hipStream_t stream) {
  using C = Fp8Cfg<D>;
  const int n_ktiles = (a.Nk + C::kBC - 1) / C::kBC;
  hipLaunchKernelGGL((fp8_vt_kernel<D>), dim3(n_ktiles, a.B * a.Hkv), dim3(256), 0, stream, (const uint8_t*)a.v,
                     (uint8_t*)a.workspace, a.Nk, n_ktiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Fp8Params p;
  p.q = (const uint8_t*)a.q; p.k = (const uint8_t*)a.k; p.vt = (const uint8_t*)a.workspace;
  p.o = a.o; p.lse = a.lse;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk; p.n_ktiles = n_ktiles;
  const ExpScale es = exp_scale(a.scale * a.q_descale * a.k_descale * kLog2e);
  p.c = es.c; p.neg_q = es.neg_q;
  p.v_descale = a.v_descale;
  const unsigned grid = (unsigned)((a.Nq + C::kBR - 1) / C::kBR) * a.B * a.Hq;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3(grid), dim3(64 * C::kWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t fp8_vt_bytes(int B, int Hkv, int Nk, int d) {
  return (size_t)B * Hkv * ((Nk + kVtKeys - 1) / kVtKeys) * kVtKeys * d;
}

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return a.causal ? launch_typed<64, true>(a, stream) : launch_typed<64, false>(a, stream);
    case 128: return a.causal ? launch_typed<128, true>(a, stream) : launch_typed<128, false>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
