// fa_fwd.hip -- exact attention forward for gfx950.
//
// Tiled attention with an online softmax (tutorial "FlashAttention and
// efficient attention kernels": sections "Online softmax", "Correction
// formula", "Forward" and the forward pseudocode skeleton; concept page
// "Flash-Attention", section "Core idea": Q outer, K/V inner, running max /
// sum / output, the N x N scores never leave the chip).
//
// Work decomposition (MI355X): one work-group of 4 waves owns 128 query rows
// of one (batch, query head); each wave owns 32 of them, so no reduction ever
// crosses waves.  The work-group streams the K/V head in tiles of kBC keys
// through LDS (double-buffered, bounds-checked direct-to-LDS buffer loads).
// Per tile each wave computes
//   S^T = K_j Q^T            (kBC x 32, 32x32x16 MFMA, fp32 accumulation)
//   online softmax in the log2 domain: one cross-lane max exchange per tile,
//   P^T = exp2(S^T * scale*log2e - m)
//   O^T = O^T * exp2(m_old - m_new) + V_j^T P^T   (P^T rounded to T, straight
//                                                   from registers)
// Lane l always holds query l % 32, so the running max/sum are per lane.
// The final O = O^T / l and LSE = (m + log2 l) * ln 2 are written once.
#include "fa_device.hpp"
#include "fa_kernels.h"

namespace fa {
namespace {

template <typename T, int D>
struct FwdCfg {
  static constexpr int kWaves = 4;
  static constexpr int kBR = 32 * kWaves;                    // query rows per work-group
  static constexpr int kES = Elem<T>::kBytes;
  static constexpr int kRowBytes = D * kES;
  static constexpr int kBC = (kES == 4 && D == 128) ? 32 : 64;  // keys per KV tile
  static constexpr int kKS = D / 16;                         // 16-wide k blocks along d
  static constexpr int kMT = kBC / 32;                       // 32-key M tiles of S^T
  static constexpr int kPS = kBC / 16;                       // 16-key k blocks of V^T P^T
  static constexpr int kDT = D / 32;                         // 32-row M tiles of O^T
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kLds = 2 * 2 * kTileBytes;            // {K, V} x double buffer
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk;
  int n_qtiles;
  float c;  // scale * log2(e)
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_kernel(FwdParams p) {
  using C = FwdCfg<T, D>;
  using E = Elem<T>;
  using F = Frags<T>;
  using TT = Tile<C::kRowBytes>;
  typedef typename E::Frag Frag;

  __shared__ __attribute__((aligned(1024))) char smem_raw[C::kLds];
  lds_char* smem = (lds_char*)smem_raw;

  // Block -> (query tile, batch, head).  With the causal mask the last query
  // tiles carry the most work, so they are dispatched first.
  const int bh_count = p.B * p.Hq;
  const int id = blockIdx.x;
  const int bh = id % bh_count;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - id / bh_count) : id / bh_count;
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);

  const int lane = lane_id(), w = wave_id();
  const int h = lane >> 5, col = lane & 31;
  const int q0 = qt * C::kBR;
  const int qw = q0 + 32 * w;  // first query row of this wave
  const int qrow = qw + col;   // this lane's query row
  const int diag = p.Nk - p.Nq;  // key j is visible to row i iff j <= i + diag (causal)

  const size_t q_slab = (size_t)bh * p.Nq * D;
  const size_t kv_slab = ((size_t)b * p.Hkv + hkv) * p.Nk * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + q_slab * C::kES, (uint32_t)p.Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.k + kv_slab * C::kES, (uint32_t)p.Nk * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)p.v + kv_slab * C::kES, (uint32_t)p.Nk * C::kRowBytes);

  int n_tiles = (p.Nk + C::kBC - 1) / C::kBC;
  if (CAUSAL) {
    const int last_key = min(q0 + C::kBR, p.Nq) - 1 + diag;
    n_tiles = last_key < 0 ? 0 : min(n_tiles, last_key / C::kBC + 1);
  }

  // Stage K/V tile j into LDS buffer `buf` (keys past Nk read as zero).
  auto load_tile = [&](int j, int buf) {
    lds_char* kb = smem + buf * 2 * C::kTileBytes;
    const uint32_t g0 = (uint32_t)j * C::kBC * C::kRowBytes;
    dma_tile<C::kRowBytes, C::kBC, C::kWaves>(rk, g0, kb, w, lane);
    dma_tile<C::kRowBytes, C::kBC, C::kWaves>(rv, g0, kb + C::kTileBytes, w, lane);
  };

  if (n_tiles > 0) load_tile(0, 0);

  // Q^T as the B operand of S^T = K Q^T: lane holds row qrow, d = 16ks + 8h + 0..7.
  Frag qf[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ks++) qf[ks] = F::template global_row<D>(rq, qrow, ks, h);

  f32x16 o[C::kDT];
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++) o[dt] = f32x16{};
  float m = -INFINITY;  // running max of scale*log2e*s (log2 domain)
  float l = 0.f;        // this lane's share of the running sum (the other half-wave holds the rest)
  const bool fast_ok = p.c > 0.f;

  wait_vmem();
  __syncthreads();

  for (int j = 0; j < n_tiles; j++) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1, buf ^ 1);
    const lds_char* kb = smem + buf * 2 * C::kTileBytes;
    const lds_char* vb = kb + C::kTileBytes;
    const int k0 = j * C::kBC;

    // A wave whose rows all end before this tile skips it (it still joins the barrier).
    if (!CAUSAL || k0 <= qw + 31 + diag) {
      // ---- S^T = K_j Q^T; A rows are sigma-permuted keys.
      f32x16 s[C::kMT];
#pragma unroll
      for (int mt = 0; mt < C::kMT; mt++) s[mt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::kKS; ks++) {
#pragma unroll
        for (int mt = 0; mt < C::kMT; mt++) {
          const Frag a = F::template lds_row<TT>(kb, 32 * mt + sigma(col), ks, h);
          s[mt] = E::mma(a, qf[ks], s[mt]);
        }
      }

      // ---- online softmax.  Register r of M tile mt holds key
      //      k0 + 32*mt + 16*(r/8) + 8h + (r%8) for query qrow.
      const bool need_mask = !fast_ok || (k0 + C::kBC > p.Nk) || (CAUSAL && k0 + C::kBC - 1 > qw + diag);
      float m_new, m_use;
      if (!need_mask) {
        float mx = s[0][0];
#pragma unroll
        for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
          for (int r = 0; r < 16; r++) mx = fmaxf(mx, s[mt][r]);
        mx = fmaxf(mx, xor32(mx));
        m_new = fmaxf(m, mx * p.c);
        m_use = m_new;
#pragma unroll
        for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
          for (int r = 0; r < 16; r++) s[mt][r] = fast_exp2(fmaf(s[mt][r], p.c, -m_use));
      } else {
        float mx = -INFINITY;
        const int horizon = CAUSAL ? min(qrow + diag, p.Nk - 1) : p.Nk - 1;
#pragma unroll
        for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int key = k0 + 32 * mt + 16 * (r >> 3) + 8 * h + (r & 7);
            const float t = key <= horizon ? s[mt][r] * p.c : -INFINITY;
            s[mt][r] = t;
            mx = fmaxf(mx, t);
          }
        mx = fmaxf(mx, xor32(mx));
        m_new = fmaxf(m, mx);
        m_use = m_new == -INFINITY ? 0.f : m_new;
#pragma unroll
        for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
          for (int r = 0; r < 16; r++) s[mt][r] = fast_exp2(s[mt][r] - m_use);
      }
      const float alpha = fast_exp2(m - m_use);  // 0 on the first visible tile
      m = m_new;
      float rs = 0.f;
#pragma unroll
      for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
        for (int r = 0; r < 16; r++) rs += s[mt][r];
      l = l * alpha + rs;
      if (!__all(alpha == 1.f)) {
#pragma unroll
        for (int dt = 0; dt < C::kDT; dt++) o[dt] *= alpha;
      }

      // ---- O^T += V_j^T P^T.  P^T k block ps = registers 8*(ps%2).. of tile ps/2.
#pragma unroll
      for (int ps = 0; ps < C::kPS; ps++) {
        float pv[8];
#pragma unroll
        for (int t = 0; t < 8; t++) pv[t] = s[ps >> 1][8 * (ps & 1) + t];
        const Frag pf = E::pack(pv);
#pragma unroll
        for (int dt = 0; dt < C::kDT; dt++) {
          const Frag a = F::template lds_col<TT>(vb, 16 * ps, 32 * dt, lane);
          o[dt] = E::mma(a, pf, o[dt]);
        }
      }
    }

    wait_vmem();
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = m + log2(l) in natural log.
  const float lt = l + xor32(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc((char*)p.o + q_slab * C::kES, (uint32_t)p.Nq * C::kRowBytes);
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++)
#pragma unroll
    for (int a4 = 0; a4 < 4; a4++) {
      const int d0 = 32 * dt + 8 * a4 + 4 * h;
      F::store4(ro, (uint32_t)qrow * C::kRowBytes + d0 * C::kES, o[dt][4 * a4] * inv, o[dt][4 * a4 + 1] * inv,
                o[dt][4 * a4 + 2] * inv, o[dt][4 * a4 + 3] * inv);
    }
  if (h == 0) {
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + (size_t)bh * p.Nq, (uint32_t)p.Nq * 4);
    const float lse = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
    buf_store4(rl, (uint32_t)qrow * 4, __builtin_bit_cast(uint32_t, lse));
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_typed(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<T, D>;
  FwdParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.lse = a.lse;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.n_qtiles = (a.Nq + C::kBR - 1) / C::kBR;
  p.c = a.scale * kLog2e;
  const unsigned grid = (unsigned)p.n_qtiles * a.B * a.Hq;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const FwdArgs& a, hipStream_t s) {
  switch (a.d) {
    case 32: return a.causal ? launch_typed<T, 32, true>(a, s) : launch_typed<T, 32, false>(a, s);
    case 64: return a.causal ? launch_typed<T, 64, true>(a, s) : launch_typed<T, 64, false>(a, s);
    case 128: return a.causal ? launch_typed<T, 128, true>(a, s) : launch_typed<T, 128, false>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 0: return launch_dtype<float>(a, stream);
    case 1: return launch_dtype<_Float16>(a, stream);
    case 2: return launch_dtype<__bf16>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
