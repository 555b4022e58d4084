// fa_fwd.hip -- exact attention forward for gfx950.
//
// Tiled attention with an online softmax (tutorial "FlashAttention and
// efficient attention kernels": sections "Online softmax", "Correction
// formula", "Forward" and the forward pseudocode skeleton; concept page
// "Flash-Attention", section "Core idea": Q outer, K/V inner, running max /
// sum / output, the N x N scores never leave the chip).
//
// Work decomposition (MI355X).  A work-group of 8 waves owns 256 query rows
// of one (batch, query head); each wave owns 32 rows, so no reduction ever
// crosses waves.  The K/V head streams through LDS in tiles of kBC keys
// (bounds-checked buffer-to-LDS loads; K and V each double-buffered).  Per
// tile j each wave computes
//   Sᵀ = K_j Qᵀ                 (kBC x 32, 32x32x16 MFMA, fp32 accumulation)
//   online softmax in the log2 domain, one cross-lane max exchange per tile,
//   Pᵀ = exp2(Sᵀ * scale*log2e - m)
//   Oᵀ = Oᵀ * exp2(m_old - m_new) + V_jᵀ Pᵀ   (Pᵀ rounded to T, straight from
//                                              registers into the next MFMA)
// Lane l always holds query l % 32, so the running max and sum are per lane;
// O = Oᵀ / l and LSE = (m + log2 l) ln 2 are written once at the end.
//
// Matrix and vector work overlap by construction ("ping-pong"): waves 0-3
// and 4-7 form two groups, and each SIMD holds one wave of each.  Time is cut
// into slots separated by work-group barriers; in a slot one group runs its
// matrix products (PV of tile j-1 and S of tile j) while the other runs the
// softmax of its last S.  Group 1 runs one slot behind group 0, so every SIMD
// always has one MFMA-phase wave and one VALU-phase wave.
//
// Grids with fewer than two 256-row work-groups per compute unit (short
// sequences, few heads) run the same kernel with 4 waves (128 rows) per
// work-group, so that the chip fills; the two groups are then waves 0-1 and
// 2-3, and a SIMD's two waves come from two work-groups.
//
// The running max moves only when a row's scores exceed it by more than 2^8
// (conditional rescaling, named on the concept page "Flash-Attention" among
// FlashAttention-4's techniques, "Known limits"); O and l share the stale max,
// so the result is unchanged while most tiles skip the rescale.
#include "fa_device.hpp"
#include "fa_kernels.h"

namespace fa {
namespace {

// Schedule of the interleaved PV/S sequence: each step is one PV product
// (two transposing reads) and one S product (one row read); the reads of the
// first PD steps go up front, then every step's products are followed by the
// reads of the step PD places later.
template <int N, int PD>
__device__ __forceinline__ void sched_pv_s() {
  constexpr int kMfma = 0x008, kDsRead = 0x100;
  constexpr int pd = PD < N ? PD : N;
  __builtin_amdgcn_sched_group_barrier(kDsRead, 3 * pd, 0);
#pragma unroll
  for (int i = 0; i < N - pd; i++) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 3, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, 2 * pd, 0);
}

template <typename T, int D, int W = 8>
struct FwdCfg {
  static constexpr int kWaves = W;                           // 8, or 4 for small grids
  static constexpr int kBR = 32 * kWaves;                    // query rows per work-group
  static constexpr int kES = Elem<T>::kBytes;
  static constexpr int kRowBytes = D * kES;
  static constexpr int kBC = (kES == 4 && D == 128) ? 32 : 64;  // keys per KV tile
  static constexpr int kKS = D / 16;                         // 16-wide k blocks along d
  static constexpr int kMT = kBC / 32;                       // 32-key M tiles of Sᵀ
  static constexpr int kPS = kBC / 16;                       // 16-key k blocks of Vᵀ Pᵀ
  static constexpr int kDT = D / 32;                         // 32-row M tiles of Oᵀ
  static constexpr int kTileBytes = kBC * kRowBytes;
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* cu_q;  // packed batch: cumulative query / key counts [B + 1], else null
  const int* cu_k;
  int B, Hq, Hkv, Nq, Nk;  // Nq, Nk: the lengths (dense) or their bounds (packed)
  int tot_q, tot_k;        // packed batch: total query / key tokens
  // Paged KV (k, v are the page caches [num_blocks, Hkv, 16, D]): the block
  // table [B, max_blocks] and cached tokens per sequence are kernel arguments
  // of their own (restrict-qualified, read through the scalar cache).
  int max_blocks, num_blocks;
  float c;    // |scale| * log2(e), or 2^-100 for a zero scale
  int neg_q;  // the scale is negative: Q's sign is flipped instead
};

constexpr float kTau = 8.0f;  // conditional-rescaling threshold (log2 units)


// PAGED: K and V are read from a paged cache through the block table; the
// queries are the last Nq positions of each sequence (dense Q, O, LSE).
template <typename T, int D, bool CAUSAL, bool PAGED, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_kernel(FwdParams p, const int* __restrict__ block_table, const int* __restrict__ seq_lens) {
  using C = FwdCfg<T, D, W>;
  using E = Elem<T>;
  using F = Frags<T>;
  using TT = Tile<C::kRowBytes>;
  typedef typename E::Frag Frag;
  constexpr bool k16 = C::kES == 2;

  // Four separate LDS objects (K and V, two buffers each): the compiler then
  // knows that a tile being loaded never aliases the tiles being read, and
  // does not make reads wait for the in-flight loads.
  __shared__ __attribute__((aligned(1024))) char k_lds0[C::kTileBytes], k_lds1[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[C::kTileBytes], v_lds1[C::kTileBytes];
  auto kbuf = [&](int par) __attribute__((always_inline)) { return (lds_char*)(par ? k_lds1 : k_lds0); };
  auto vbuf = [&](int par) __attribute__((always_inline)) { return (lds_char*)(par ? v_lds1 : v_lds0); };

  // Block -> (query tile, batch, head).  With the causal mask the last query
  // tiles carry the most work, so they are dispatched first.  The grid covers
  // the longest sequence; blocks past a shorter one's last tile leave at once.
  const int bh_count = p.B * p.Hq;
  const int id = blockIdx.x;
  const int bh = id % bh_count;
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);
  SeqRows sr;
  if constexpr (PAGED) {
    // Cached tokens of the sequence, clamped to what its table row can address.
    const int n = min(max(seq_lens[b], 0), p.max_blocks * 16);
    sr = SeqRows{p.Nq, n, b * p.Nq, 0};
  } else {
    sr = seq_rows(p.cu_q, p.cu_k, b, p.Nq, p.Nk, p.tot_q, p.tot_k);
  }
  const int Nq = sr.nq, Nk = sr.nk;
  const int n_qt = (Nq + C::kBR - 1) / C::kBR;
  if (id / bh_count >= n_qt) return;
  const int qt = CAUSAL ? (n_qt - 1 - id / bh_count) : id / bh_count;

  const int lane = lane_id(), w = wave_id();
  const int h = lane >> 5, col = lane & 31;
  const int q0 = qt * C::kBR;
  const int qw = q0 + 32 * w;     // first query row of this wave
  const int qrow = qw + col;      // this lane's query row
  const int diag = Nk - Nq;       // key j is visible to row i iff j <= i + diag (causal)

  const size_t q_row0 = (size_t)p.Hq * sr.tq + (size_t)hq * Nq;     // first row of this (sequence, head)
  const size_t kv_row0 = (size_t)p.Hkv * sr.tk + (size_t)hkv * Nk;
  const size_t q_slab = q_row0 * D;
  const size_t kv_slab = kv_row0 * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + q_slab * C::kES, (uint32_t)Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.k + kv_slab * C::kES, (uint32_t)Nk * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)p.v + kv_slab * C::kES, (uint32_t)Nk * C::kRowBytes);

  int n_tiles = (Nk + C::kBC - 1) / C::kBC;
  if (CAUSAL) {
    const int last_key = min(q0 + C::kBR, Nq) - 1 + diag;
    n_tiles = last_key < 0 ? 0 : min(n_tiles, last_key / C::kBC + 1);
  }
  // Paged KV: the rows a wave moves of any tile lie in one page; PageRef is
  // that page for one tile (byte offset of its (page, kv head) block in the
  // cache and bytes of valid rows; 0 bytes reads zeros).
  struct PageRef {
    size_t off;
    uint32_t bytes;
  };
  const int wrow0 = dma_wave_row0<C::kRowBytes, C::kBC, C::kWaves>(w);
  const int* trow = PAGED ? block_table + (size_t)b * p.max_blocks : nullptr;
  auto page_of = [&](int jj) __attribute__((always_inline)) {
    PageRef r{0, 0u};
    if constexpr (PAGED) {
      const int t0 = jj * C::kBC + wrow0;  // first token of this wave's rows
      if (jj < n_tiles && t0 < Nk) {
        const int id = trow[t0 >> 4];
        if (id >= 0 && id < p.num_blocks) {  // a bad table entry reads as a page of zeros
          r.off = ((size_t)id * p.Hkv + hkv) * (16 * C::kRowBytes);
          r.bytes = (uint32_t)min(16, Nk - (t0 & ~15)) * C::kRowBytes;
        }
      }
    }
    return r;
  };
  // Page of tile j (its V is staged one slot pair after its K) and of tile j + 1.
  PageRef pg_j = page_of(0), pg_j1 = page_of(1);
  auto dma_k = [&](int j, lds_char* dst, const PageRef& pr) __attribute__((always_inline)) {
    if constexpr (PAGED)
      dma_tile<C::kRowBytes, C::kBC, C::kWaves, true>(make_rsrc((const char*)p.k + pr.off, pr.bytes), 0u, dst, w,
                                                      lane);
    else
      dma_tile<C::kRowBytes, C::kBC, C::kWaves>(rk, (uint32_t)j * C::kBC * C::kRowBytes, dst, w, lane);
  };
  auto dma_v = [&](int j, lds_char* dst, const PageRef& pr) __attribute__((always_inline)) {
    if constexpr (PAGED)
      dma_tile<C::kRowBytes, C::kBC, C::kWaves, true>(make_rsrc((const char*)p.v + pr.off, pr.bytes), 0u, dst, w,
                                                      lane);
    else
      dma_tile<C::kRowBytes, C::kBC, C::kWaves>(rv, (uint32_t)j * C::kBC * C::kRowBytes, dst, w, lane);
  };
  if (n_tiles > 0) dma_k(0, kbuf(0), pg_j);

  // Qᵀ as the B operand of Sᵀ = K Qᵀ: lane holds row qrow, d = 16ks + 8h + 0..7.
  Frag qf[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ks++) qf[ks] = F::template global_row<D>(rq, qrow, ks, h);
  if (p.neg_q) {
#pragma unroll
    for (int ks = 0; ks < C::kKS; ks++) qf[ks] = E::negate(qf[ks]);
  }

  // Per-lane LDS offsets of the K row fragments (A rows are sigma-permuted
  // keys) and of the V column fragments; M tiles / k blocks add constants.
  uint32_t koff[k16 ? C::kKS : 1], voff[k16 ? C::kDT : 1][2];
  if constexpr (k16) {
#pragma unroll
    for (int ks = 0; ks < C::kKS; ks++) koff[ks] = F::template row_off<TT>(sigma(col), ks, h);
#pragma unroll
    for (int dt = 0; dt < C::kDT; dt++)
#pragma unroll
      for (int u = 0; u < 2; u++) voff[dt][u] = F::template col_off<TT>(32 * dt, u, lane);
  }

  f32x16 o[C::kDT];
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++) o[dt] = f32x16{};
  f32x16 s[C::kMT];     // scores of the last S, consumed by the next softmax
  Frag pf[C::kPS];      // probabilities of the last softmax, consumed by the next PV
  // 16-bit types run PV of tile j-1 and S of tile j as one sequence from tile
  // 0 on: the first one multiplies zero probabilities by a zeroed V buffer and
  // sums zero scores, so it adds nothing.
#pragma unroll
  for (int mt = 0; mt < C::kMT; mt++) s[mt] = f32x16{};
#pragma unroll
  for (int ps = 0; ps < C::kPS; ps++) pf[ps] = Frag{};
  if constexpr (k16) {
    // Zero the second K and V buffers (V(-1) of that first sequence, and the
    // K read past the last tile, whose scores are never used).
    for (int i = threadIdx.x; i < C::kTileBytes / 16; i += 64 * C::kWaves) {
      *(__attribute__((address_space(3))) u32x4*)(kbuf(1) + 16 * i) = u32x4{0, 0, 0, 0};
      *(__attribute__((address_space(3))) u32x4*)(vbuf(1) + 16 * i) = u32x4{0, 0, 0, 0};
    }
  }
  float m = -INFINITY;  // running (possibly stale) max of scale*log2e*s, log2 domain
  float l = 0.f;        // this lane's share of the running sum (the other half-wave holds the rest)
  // c > 0, so the max of c*s over a row is c*max(s).
  const float c = p.c;

  // Does this wave see any key of tile j?
  auto active = [&](int j) __attribute__((always_inline)) { return j < n_tiles && (!CAUSAL || j * C::kBC <= qw + 31 + diag); };

  // ---- the three phases --------------------------------------------------
  auto gemm_s = [&](const lds_char* kb) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++) s[mt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::kKS; ks++) {
#pragma unroll
      for (int mt = 0; mt < C::kMT; mt++) {
        Frag a;
        if constexpr (k16) a = F::lds_row_at(kb + 32 * mt * C::kRowBytes, koff[ks]);
        else a = F::template lds_row<TT>(kb, 32 * mt + sigma(col), ks, h);
        s[mt] = E::mma(a, qf[ks], s[mt]);
      }
    }
    if constexpr (k16) sched_reads_ahead<C::kKS * C::kMT, C::kKS * C::kMT, 4>();
  };
  auto gemm_pv = [&](const lds_char* vb) __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < C::kPS; ps++) {
#pragma unroll
      for (int dt = 0; dt < C::kDT; dt++) {
        Frag a;
        if constexpr (k16) a = F::lds_col_at(vb + 16 * ps * C::kRowBytes, voff[dt][0], voff[dt][1]);
        else a = F::template lds_col<TT>(vb, 16 * ps, 32 * dt, lane);
        o[dt] = E::mma(a, pf[ps], o[dt]);
      }
    }
    if constexpr (k16) sched_reads_ahead<2 * C::kPS * C::kDT, C::kPS * C::kDT, 4>();
    // Row sums of this P in float32, still in s until S of the next tile
    // overwrites it; added here because the softmax phase is the busier one.
    float rs[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
      for (int r = (mt == 0 ? 4 : 0); r < 16; r++) rs[r & 3] += s[mt][r];
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };
  // PV of the last tile and S of this tile in one interleaved sequence (16-bit
  // types): step i issues one PV and one S product (both counts equal
  // kBC*D/512), so the slower transposing V reads and the K row reads share
  // the LDS evenly instead of arriving in two bursts.  The row sums of the
  // last P are taken from s first, so the new S can take its registers.
  auto gemm_fused = [&](const lds_char* vb, const lds_char* kb) __attribute__((always_inline)) {
    if constexpr (k16) {
    constexpr int N = C::kPS * C::kDT;
    static_assert(N == C::kKS * C::kMT, "PV and S have equal product counts");
    float rs[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
      for (int r = (mt == 0 ? 4 : 0); r < 16; r++) rs[r & 3] += s[mt][r];
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++) s[mt] = f32x16{};
#pragma unroll
    for (int i = 0; i < N; i++) {
      const int ps = i / C::kDT, dt = i % C::kDT;
      const Frag av = F::lds_col_at(vb + 16 * ps * C::kRowBytes, voff[dt][0], voff[dt][1]);
      o[dt] = E::mma(av, pf[ps], o[dt]);
      const int ks = i / C::kMT, mt = i % C::kMT;
      const Frag ak = F::lds_row_at(kb + 32 * mt * C::kRowBytes, koff[ks]);
      s[mt] = E::mma(ak, qf[ks], s[mt]);
    }
    sched_pv_s<N, 3>();
    }
  };
  // Register r of M tile mt holds key k0 + 32*mt + 16*(r/8) + 8h + (r%8).
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * C::kBC;
    // Invisible keys (past Nk, past the causal horizon) get score -inf; the
    // rest of the softmax is one code path for every tile.
    if ((k0 + C::kBC > Nk) || (CAUSAL && k0 + C::kBC - 1 > qw + diag)) {
      const int horizon = CAUSAL ? min(qrow + diag, Nk - 1) : Nk - 1;
#pragma unroll
      for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int key = k0 + 32 * mt + 16 * (r >> 3) + 8 * h + (r & 7);
          if (key > horizon) s[mt][r] = -INFINITY;
        }
    }
    // Four independent three-input max chains; c > 0, so max(c s) = c max(s).
    float x[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
      for (int r = (mt == 0 ? 4 : 0); r < 16; r += 8)
#pragma unroll
        for (int i = 0; i < 4; i++)
          x[i] = r + 4 + i < 16 ? vmax(vmax(x[i], s[mt][r + i]), s[mt][r + 4 + i]) : vmax(x[i], s[mt][r + i]);
    const float mx = max_halves(vmax(vmax(x[0], x[1]), vmax(x[2], x[3]))) * c;
    // Move the running max only if it grows by more than kTau.
    const bool grow = mx > m + kTau;
    if (__any(grow)) {
      // 1 where the max stays (also rows that have seen no key yet), 0 on a row's first keys.
      const float alpha = grow ? fast_exp2(m - mx) : 1.f;
      m = grow ? mx : m;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::kDT; dt++) o[dt] *= alpha;
    }
    const float m_use = m == -INFINITY ? 0.f : m;  // rows that have seen no key yet
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) s[mt][r] = fast_exp2(fmaf(s[mt][r], c, -m_use));
    // (The row sums of P are added in the next PV phase.)
    // Pᵀ k block ps = registers 8*(ps%2).. of tile ps/2.
#pragma unroll
    for (int ps = 0; ps < C::kPS; ps++) {
      float pv[8];
#pragma unroll
      for (int t = 0; t < 8; t++) pv[t] = s[ps >> 1][8 * (ps & 1) + t];
      pf[ps] = E::pack(pv);
    }
  };

  // ---- slot schedule -----------------------------------------------------
  // Slot t (one barrier after each): loads of K(t/2 + 1) and V(t/2) are issued
  // in even slots and waited for at the end of the next (odd) slot.  A wave
  // of group G runs phase u = t - G: even u = GEMM of tile u/2 (PV of tile
  // u/2 - 1, then S of tile u/2), odd u = softmax of tile (u-1)/2.  Slots
  // are unrolled by 4 so every buffer parity is a compile-time constant.
  const int G = w / (C::kWaves / 2);
  const int n_slots = (2 * n_tiles + 2 + 3) & ~3;

  auto slot = [&](auto gc, auto pc, int t) __attribute__((always_inline)) {
    constexpr int g = decltype(gc)::value, p4 = decltype(pc)::value;
    if constexpr ((p4 & 1) == 0) {
      const int j = t >> 1;
      constexpr int jp = (p4 >> 1) & 1;  // parity of j
      if (j + 1 < n_tiles) dma_k(j + 1, kbuf(jp ^ 1), pg_j1);
      if (j < n_tiles) dma_v(j, vbuf(jp), pg_j);
    }
    const int u = t - g;
    if (u >= 0) {
      if constexpr (((p4 - g) & 1) == 0) {
        const int j = u >> 1;
        constexpr int jp = ((p4 - g + 4) >> 1) & 1;  // parity of j
        // active() is monotone in j for a wave (tile j active implies tile j-1
        // active), so this runs PV(j-1) whenever it is due and S(j) with it.
        if (k16) {
          // The matrix phase runs at raised wave priority, so that its MFMA
          // and LDS instructions win issue arbitration over the softmax wave
          // on the same SIMD.
          if (j == 0 ? active(0) : active(j - 1)) {
            __builtin_amdgcn_s_setprio(3);
            gemm_fused(vbuf(jp ^ 1), kbuf(jp));
            __builtin_amdgcn_s_setprio(0);
          }
        } else {
          if (j >= 1 && active(j - 1)) gemm_pv(vbuf(jp ^ 1));
          // s is (re)defined on both paths, so the probabilities left in it by
          // the last softmax are dead after PV: a tile that skips S also skips
          // its softmax, so any value will do.
          if (active(j)) gemm_s(kbuf(jp));
          else {
#pragma unroll
            for (int mt = 0; mt < C::kMT; mt++) s[mt] = __builtin_nondeterministic_value(s[mt]);
          }
        }
      } else {
        const int j = (u - 1) >> 1;
        if (active(j)) softmax(j);
      }
    }
    // Odd slots end the tile: the loads issued in the even slot have landed
    // (each wave waits for its own) and every wave is done with the buffers
    // that the next even slot refills.  The even slots need no barrier.
    if constexpr (p4 & 1) {
      if constexpr (PAGED) {
        // Table entries for the next even slot, read after this slot's LDS
        // work (the empty asm keeps them there) so that their wait merges
        // with the barrier's.
        asm volatile("" ::: "memory");
        pg_j = pg_j1;
        pg_j1 = page_of((t >> 1) + 2);
      }
      wait_vmem();
      barrier_lds();
    }
  };

  wait_vmem();
  barrier_lds();
  auto run = [&](auto gc) __attribute__((always_inline)) {
    for (int t = 0; t < n_slots; t += 4) {
      slot(gc, Int<0>{}, t);
      slot(gc, Int<1>{}, t + 1);
      slot(gc, Int<2>{}, t + 2);
      slot(gc, Int<3>{}, t + 3);
    }
  };
  if (G == 0) run(Int<0>{});
  else run(Int<1>{});

  // ---- epilogue: O = Oᵀ / l, LSE = m + log2(l) in natural log.
  const float lt = sum_halves(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc((char*)p.o + q_slab * C::kES, (uint32_t)Nq * C::kRowBytes);
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++)
#pragma unroll
    for (int a4 = 0; a4 < 4; a4++) {
      const int d0 = 32 * dt + 8 * a4 + 4 * h;
      F::store4(ro, (uint32_t)qrow * C::kRowBytes + d0 * C::kES, o[dt][4 * a4] * inv, o[dt][4 * a4 + 1] * inv,
                o[dt][4 * a4 + 2] * inv, o[dt][4 * a4 + 3] * inv);
    }
  if (h == 0) {
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + q_row0, (uint32_t)Nq * 4);
    const float lse = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
    buf_store4(rl, (uint32_t)qrow * 4, __builtin_bit_cast(uint32_t, lse));
  }
}

template <typename T, int D, bool CAUSAL, bool PAGED, int W>
hipError_t launch_typed(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<T, D, W>;
  FwdParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.lse = a.lse;
  p.cu_q = a.cu_q; p.cu_k = a.cu_k;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.tot_q = a.tot_q; p.tot_k = a.tot_k;
  p.max_blocks = a.max_blocks; p.num_blocks = a.num_blocks;
  const ExpScale es = exp_scale(a.scale * kLog2e);
  p.c = es.c; p.neg_q = es.neg_q;
  const unsigned grid = (unsigned)((a.Nq + C::kBR - 1) / C::kBR) * a.B * a.Hq;
  if (grid == 0) return hipSuccess;  // a packed batch with no query
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, PAGED, W>), dim3(grid), dim3(64 * C::kWaves), 0, stream, p,
                     a.block_table, a.seq_lens);
  return hipGetLastError();
}

template <typename T, int D, int W>
hipError_t launch_mask(const FwdArgs& a, hipStream_t s) {
  if (a.block_table)
    return a.causal ? launch_typed<T, D, true, true, W>(a, s) : launch_typed<T, D, false, true, W>(a, s);
  return a.causal ? launch_typed<T, D, true, false, W>(a, s) : launch_typed<T, D, false, false, W>(a, s);
}

// 8-wave work-groups unless that grid gives fewer than two per compute unit
// of the device.  Such short grids run, for 16-bit types, the kernel whose
// two wave groups split each 128-row tile's keys (half the serial chain of
// tiles per work-group, the ping-pong kept); float32 runs the 4-wave
// instance of this kernel.
template <typename T, int D>
hipError_t launch_waves(const FwdArgs& a, hipStream_t s) {
  const int64_t grid8 = (int64_t)((a.Nq + FwdCfg<T, D, 8>::kBR - 1) / FwdCfg<T, D, 8>::kBR) * a.B * a.Hq;
  if (grid8 >= 2 * (int64_t)a.cus) return launch_mask<T, D, 8>(a, s);
  if constexpr (Elem<T>::kBytes == 2) return launch_fwd_keysplit(a, s);
  else return launch_mask<T, D, 4>(a, s);
}

template <typename T>
hipError_t launch_dtype(const FwdArgs& a, hipStream_t s) {
  switch (a.d) {
    case 32: return launch_waves<T, 32>(a, s);
    case 64: return launch_waves<T, 64>(a, s);
    case 128: return launch_waves<T, 128>(a, s);
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
