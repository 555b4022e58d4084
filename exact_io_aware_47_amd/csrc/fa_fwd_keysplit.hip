// fa_fwd_keysplit.hip -- exact attention forward for gfx950, with the key
// range of a query tile split between the two wave groups of a work-group.
//
// Same method as fa_fwd.hip (tutorial "FlashAttention and efficient
// attention kernels": "Online softmax", "Correction formula", "Forward";
// concept page "Flash-Attention", "Core idea"), combined with the split of
// the key sequence that the tutorial's "Variant family" section describes for
// FlashDecoding: partial softmax results over disjoint key ranges, merged
// with the correction formula.  Two kernels: fwd_keysplit_kernel (8 waves,
// slot schedule) below, and fwd_keysplit_plain_kernel (4 waves, no slot
// schedule, causal calls with head sizes up to 64) further down.
//
// Work decomposition.  A work-group of 8 waves owns kBR = 4 * RW query rows
// of one (batch, query head).  Waves w and w + 4 (the same SIMD) own the same
// RW rows: wave group 0 (waves 0-3) takes the key tiles 0, 2, 4, ... and
// group 1 (waves 4-7) the tiles 1, 3, 5, ..., each with its own running
// (max, sum, output).  At the end group 1 hands its partial results to
// group 0 through LDS, which merges them (M = max(m0, m1),
// l = l0 2^(m0-M) + l1 2^(m1-M), O likewise) and writes O and LSE.
//
// Time is cut into slots with one work-group barrier each.  In slot t the
// group whose tiles have t's parity runs its matrix phase (Oᵀ += Vᵀ Pᵀ of its
// previous tile t - 2, then Sᵀ = K Qᵀ of tile t) while the other group runs
// the softmax of the tile it multiplied in slot t - 1, so each SIMD holds one
// MFMA-phase and one VALU-phase wave ("ping-pong").  Slot t reads K(t) and
// V(t - 2) and loads K(t + 1) and V(t - 1) into the other buffers.
//
// K and V come from contiguous tensors (dense or packed batches) or, with
// PAGED, from 16-token pages through the block table, staged page by page
// as in fa_fwd.hip.  Each wave owns 32 rows and each tile 64 keys, as in the
// 8-wave kernel of fa_fwd.hip; the difference is that a work-group covers 128 rows and takes
// one tile per slot instead of one per two slots.  For grids with fewer than
// two 256-row work-groups per compute unit this halves the serial chain of
// tiles of a work-group while keeping the ping-pong (the 4-wave instance of
// the 8-wave kernel has no partner wave on a SIMD).
//
// Layouts and the softmax follow fa_fwd.hip: queries on lanes (column of the
// 32x32x16 product), the sigma row order that puts Pᵀ straight into the
// B-operand layout, exp2 with scale*log2(e) folded into one FMA, and a
// running max that moves only when it grows by more than 2^8.
#include "fa_device.hpp"
#include "fa_kernels.h"

namespace fa {
namespace {

template <typename T, int D>
struct KsCfg {
  static constexpr int kWaves = 8;
  static constexpr int kBR = 128;                          // query rows per work-group (32 per wave)
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBC = 64;                           // keys per tile
  static constexpr int kKS = D / 16;                       // 16-wide k blocks along d
  static constexpr int kMT = kBC / 32;                     // 32-key M tiles of Sᵀ
  static constexpr int kPS = kBC / 16;                     // 16-key k blocks of Vᵀ Pᵀ
  static constexpr int kDT = D / 32;                       // 32-row M tiles of Oᵀ
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kOFloats = kDT * 16;                // O accumulator floats per lane
};

struct KsParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* cu_q;  // packed batch: cumulative query / key counts [B + 1], else null
  const int* cu_k;
  int B, Hq, Hkv, Nq, Nk;
  int tot_q, tot_k;
  // Paged KV (k, v are the page caches [num_blocks, Hkv, 16, D]): the block
  // table [B, max_blocks] and cached tokens per sequence are kernel arguments
  // of their own (restrict-qualified, read through the scalar cache).
  int max_blocks, num_blocks;
  float c;    // |scale| * log2(e), or 2^-100 for a zero scale
  int neg_q;  // the scale is negative: Q's sign is flipped instead
};

constexpr float kTau = 8.0f;  // conditional-rescaling threshold (log2 units)

// Schedule of NU fragment reads of RPU LDS instructions each, every fragment
// feeding MPU MFMAs: the first PD fragments are read up front, then every
// fragment's products are followed by the reads of the fragment PD places
// later.
template <int NU, int RPU, int MPU, int PD>
__device__ __forceinline__ void sched_units() {
  constexpr int kMfma = 0x008, kDsRead = 0x100;
  constexpr int pd = PD < NU ? PD : NU;
  __builtin_amdgcn_sched_group_barrier(kDsRead, RPU * pd, 0);
#pragma unroll
  for (int i = 0; i < NU - pd; i++) {
    __builtin_amdgcn_sched_group_barrier(kMfma, MPU, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, RPU, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, MPU * pd, 0);
}

// PAGED: K and V are read from a paged cache through the block table; the
// queries are the last Nq positions of each sequence (dense Q, O, LSE).
template <typename T, int D, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_keysplit_kernel(KsParams p, const int* __restrict__ block_table, const int* __restrict__ seq_lens) {
  using C = KsCfg<T, D>;
  using E = Elem<T>;
  using F = Frags<T>;
  using TT = Tile<C::kRowBytes>;
  typedef typename E::Frag Frag;
  constexpr int KS = C::kKS, MT = C::kMT, PS = C::kPS, DT = C::kDT;

  __shared__ __attribute__((aligned(1024))) char k_lds0[C::kTileBytes], k_lds1[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[C::kTileBytes], v_lds1[C::kTileBytes];
  // Merge area: per group-0 wave, its partner's O floats (16-byte groups,
  // lane-major) and its running max and sum.
  __shared__ __attribute__((aligned(1024))) char mg_lds[4 * C::kOFloats * 64 * 4];
  __shared__ __attribute__((aligned(1024))) char st_lds[4 * 2 * 64 * 4];
  auto kbuf = [&](int par) __attribute__((always_inline)) { return (lds_char*)(par ? k_lds1 : k_lds0); };
  auto vbuf = [&](int par) __attribute__((always_inline)) { return (lds_char*)(par ? v_lds1 : v_lds0); };

  // Block -> (query tile, batch, head); causal: the heaviest tiles first.
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
  const int G = w >> 2, wl = w & 3;  // wave group, wave within the group
  const int h = lane >> 5, col = lane & 31;
  const int q0 = qt * C::kBR;
  const int qw = q0 + 32 * wl;       // first query row of this wave
  const int qrow = qw + col;         // this lane's query row
  const int diag = Nk - Nq;          // key j is visible to row i iff j <= i + diag (causal)

  const size_t q_row0 = (size_t)p.Hq * sr.tq + (size_t)hq * Nq;
  const size_t kv_row0 = (size_t)p.Hkv * sr.tk + (size_t)hkv * Nk;
  const size_t q_slab = q_row0 * D;
  const size_t kv_slab = kv_row0 * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + q_slab * 2, (uint32_t)Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.k + kv_slab * 2, (uint32_t)Nk * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)p.v + kv_slab * 2, (uint32_t)Nk * C::kRowBytes);

  int n_tiles = (Nk + C::kBC - 1) / C::kBC;
  if (CAUSAL) {
    const int last_key = min(q0 + C::kBR, Nq) - 1 + diag;
    n_tiles = last_key < 0 ? 0 : min(n_tiles, last_key / C::kBC + 1);
  }
  // Paged KV: the rows a wave moves of any tile lie in one 16-token page;
  // PageRef is that page for one tile (byte offset of its (page, kv head)
  // block in the cache and bytes of valid rows; 0 bytes reads zeros).
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
      if (jj >= 0 && jj < n_tiles && t0 < Nk) {
        const int pid = trow[t0 >> 4];
        if (pid >= 0 && pid < p.num_blocks) {  // a bad table entry reads as a page of zeros
          r.off = ((size_t)pid * p.Hkv + hkv) * (16 * C::kRowBytes);
          r.bytes = (uint32_t)min(16, Nk - (t0 & ~15)) * C::kRowBytes;
        }
      }
    }
    return r;
  };
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
  // Pages of the tiles the next slot loads: K(t + 1) and V(t - 1) for slot t.
  PageRef pg_k = page_of(1), pg_v = page_of(-1);
  if (n_tiles > 0) dma_k(0, kbuf(0), page_of(0));

  // Qᵀ as the B operand of Sᵀ = K Qᵀ: lane holds row qrow, d = 16ks + 8h + 0..7.
  Frag qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    qf[ks] = F::template global_row<D>(rq, qrow, ks, h);
    if (p.neg_q) qf[ks] = E::negate(qf[ks]);
  }

  // Per-lane LDS offsets of the K row fragments (A rows are sigma-permuted
  // keys) and of the Vᵀ column fragments.  The tile swizzle XORs a row's
  // 16-byte chunk index with a per-row key, and row offsets are multiples of
  // the row size (a power of two above every chunk offset used), so fragment
  // ks of K lies at kbase ^ 32 ks and column tile dt of Vᵀ at
  // vbase[u] ^ 64 dt: three registers and one XOR per read instead of one
  // register per fragment.
  uint32_t kbase = F::template row_off<TT>(sigma(col), 0, h);
  uint32_t vbase[2] = {F::template col_off<TT>(0, 0, lane), F::template col_off<TT>(0, 1, lane)};

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) o[dt] = f32x16{};
  f32x16 s[MT];   // scores of this group's current tile
  Frag pf[PS];    // its probabilities, consumed by the next matrix phase
  float m = -INFINITY;  // running (possibly stale) max of scale*log2e*s, log2 domain
  float l = 0.f;        // this lane's share of the running sum
  const float c = p.c;  // > 0, so the max of c*s over a row is c*max(s)

  // Does this wave see any key of tile j?
  auto active = [&](int j) __attribute__((always_inline)) {
    return j >= 0 && j < n_tiles && (!CAUSAL || j * C::kBC <= qw + 31 + diag);
  };

  auto gemm_pv = [&](const lds_char* vb) __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < PS; ps++)
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        const Frag a = F::lds_col_at(vb + 16 * ps * C::kRowBytes, vbase[0] ^ (uint32_t)(64 * dt),
                                     vbase[1] ^ (uint32_t)(64 * dt));
        o[dt] = E::mma(a, pf[ps], o[dt]);
      }
    sched_units<PS * DT, 2, 1, 2>();
  };
  auto gemm_s = [&](const lds_char* kb) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++) s[mt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const Frag a = F::lds_row_at(kb + 32 * mt * C::kRowBytes, kbase ^ (uint32_t)(32 * ks));
        s[mt] = E::mma(a, qf[ks], s[mt]);
      }
    sched_units<KS * MT, 1, 1, 2>();
  };
  // Register r of M tile mt holds key k0 + 32*mt + 16*(r/8) + 8h + (r%8).
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * C::kBC;
    if ((k0 + C::kBC > Nk) || (CAUSAL && k0 + C::kBC - 1 > qw + diag)) {
      const int horizon = CAUSAL ? min(qrow + diag, Nk - 1) : Nk - 1;
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int key = k0 + 32 * mt + 16 * (r >> 3) + 8 * h + (r & 7);
          if (key > horizon) s[mt][r] = -INFINITY;
        }
    }
    // Four independent three-input max chains; c > 0, so max(c s) = c max(s).
    float x[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int r = (mt == 0 ? 4 : 0); r < 16; r += 8)
#pragma unroll
        for (int i = 0; i < 4; i++)
          x[i] = r + 4 + i < 16 ? vmax(vmax(x[i], s[mt][r + i]), s[mt][r + 4 + i]) : vmax(x[i], s[mt][r + i]);
    const float mx = max_halves(vmax(vmax(x[0], x[1]), vmax(x[2], x[3]))) * c;
    // Move the running max only if it grows by more than kTau.
    const bool grow = mx > m + kTau;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m - mx) : 1.f;
      m = grow ? mx : m;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; dt++) o[dt] *= alpha;
    }
    const float m_use = m == -INFINITY ? 0.f : m;  // rows that have seen no key yet
    float rs[4];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        s[mt][r] = fast_exp2(fmaf(s[mt][r], c, -m_use));
        rs[r & 3] = (mt == 0 && r < 4) ? s[mt][r] : rs[r & 3] + s[mt][r];
      }
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    // Pᵀ k block ps = registers 8*(ps%2).. of M tile ps/2.
#pragma unroll
    for (int ps = 0; ps < PS; ps++) {
      float pv[8];
#pragma unroll
      for (int t = 0; t < 8; t++) pv[t] = s[ps >> 1][8 * (ps & 1) + t];
      pf[ps] = E::pack(pv);
    }
  };

  // ---- slot schedule (one barrier per slot).  Slot t: loads of K(t + 1)
  // and V(t - 1); the group of parity t runs its matrix phase (PV of tile
  // t - 2, S of tile t), the other group the softmax of tile t - 1.  Slots are
  // unrolled by two so that every buffer is a compile-time object, and each
  // group runs its own copy of the loop, so every slot is straight-line code.
  const int n_slots = n_tiles + 2;
  auto slot = [&](auto gc, auto pc, int t) __attribute__((always_inline)) {
    constexpr int g = decltype(gc)::value;    // this wave's group
    constexpr int par = decltype(pc)::value;  // parity of t
    // The lane offsets are re-hidden from the compiler at every slot, so
    // that it adds them to the buffer bases inside the slot instead of
    // keeping one hoisted address register per (buffer, fragment) pair.
    asm volatile("" : "+v"(kbase), "+v"(vbase[0]), "+v"(vbase[1]));
    if (t + 1 < n_tiles) dma_k(t + 1, kbuf(par ^ 1), pg_k);
    if (t >= 1 && t - 1 < n_tiles) dma_v(t - 1, vbuf(par ^ 1), pg_v);
    if constexpr (g == par) {
      if (active(t - 2)) gemm_pv(vbuf(par));
      if (active(t)) gemm_s(kbuf(par));
    } else {
      if (active(t - 1)) softmax(t - 1);
    }
    if constexpr (PAGED) {
      // Table entries of the next slot's tiles, read after this slot's LDS
      // work (the empty asm keeps them there) so that their wait merges with
      // the barrier's.
      asm volatile("" ::: "memory");
      pg_k = page_of(t + 2);
      pg_v = page_of(t);
    }
    wait_vmem();
    barrier_lds();
  };
  wait_vmem();
  barrier_lds();
  auto run = [&](auto gc) __attribute__((always_inline)) {
    for (int t = 0; t < n_slots; t += 2) {
      slot(gc, Int<0>{}, t);
      slot(gc, Int<1>{}, t + 1);
    }
  };
  if (G == 0) run(Int<0>{});
  else run(Int<1>{});

  // ---- merge: group 1 hands (O, m, l) to the group-0 wave with its rows;
  // that wave rescales both parts to the common max and adds them.
  lds_char* const mg = (lds_char*)mg_lds + wl * C::kOFloats * 64 * 4;
  __attribute__((address_space(3))) float* const st =
      (__attribute__((address_space(3))) float*)((lds_char*)st_lds + wl * 2 * 64 * 4);
  if (G == 1) {
    st[lane] = m;
    st[64 + lane] = l;
#pragma unroll
    for (int f4 = 0; f4 < C::kOFloats / 4; f4++) {
      const int dt = f4 / 4, r = 4 * (f4 % 4);
      *(__attribute__((address_space(3))) f32x4*)(mg + (f4 * 64 + lane) * 16) =
          f32x4{o[dt][r], o[dt][r + 1], o[dt][r + 2], o[dt][r + 3]};
    }
  }
  barrier_lds();
  if (G == 1) return;
  {
    const float m1 = st[lane], l1 = st[64 + lane];
    const float M = vmax(m, m1);
    const float a0 = m == -INFINITY ? 0.f : fast_exp2(m - M);
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - M);
    l = a0 * l + a1 * l1;
    m = M;
#pragma unroll
    for (int f4 = 0; f4 < C::kOFloats / 4; f4++) {
      const int dt = f4 / 4, r = 4 * (f4 % 4);
      const f32x4 v4 = *(__attribute__((address_space(3))) f32x4*)(mg + (f4 * 64 + lane) * 16);
#pragma unroll
      for (int i = 0; i < 4; i++) o[dt][r + i] = fmaf(a1, v4[i], a0 * o[dt][r + i]);
    }
  }

  // ---- epilogue (group 0): O = Oᵀ / l, LSE = m + log2(l) in natural log.
  const float lt = sum_halves(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc((char*)p.o + q_slab * 2, (uint32_t)Nq * C::kRowBytes);
#pragma unroll
  for (int dt = 0; dt < DT; dt++)
#pragma unroll
    for (int a4 = 0; a4 < 4; a4++) {
      const int d0 = 32 * dt + 8 * a4 + 4 * h;
      F::store4(ro, (uint32_t)qrow * C::kRowBytes + d0 * 2, o[dt][4 * a4] * inv, o[dt][4 * a4 + 1] * inv,
                o[dt][4 * a4 + 2] * inv, o[dt][4 * a4 + 3] * inv);
    }
  if (h == 0) {
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + q_row0, (uint32_t)Nq * 4);
    const float lse = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
    buf_store4(rl, (uint32_t)qrow * 4, __builtin_bit_cast(uint32_t, lse));
  }
}

// ---------------------------------------------------------------------------
// The same key split without the slot schedule, for causal grids with head
// sizes up to 64.  A
// work-group of 4 waves owns 64 query rows: waves 0-1 (group 0) take the even
// key tiles and waves 2-3 (group 1) the odd ones, as above, each group with
// its own double-buffered K and V tiles, and every wave runs S, the softmax
// and PV of its tile in turn.  The grid has twice the work-groups of the
// 8-wave kernel, and two of them share a compute unit: the two waves of a
// SIMD then come from different work-groups and run out of step, so one's
// products overlap the other's softmax without a barrier-paced alternation.
// Every tile's arithmetic and the merge are those of fwd_keysplit_kernel, in
// the same order, so the two kernels give bitwise-equal results.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct KpCfg {
  static constexpr int kWaves = 4;
  static constexpr int kBR = 64;                           // query rows per work-group (32 per wave)
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBC = 64;                           // keys per tile
  static constexpr int kKS = D / 16;                       // 16-wide k blocks along d
  static constexpr int kMT = kBC / 32;                     // 32-key M tiles of Sᵀ
  static constexpr int kPS = kBC / 16;                     // 16-key k blocks of Vᵀ Pᵀ
  static constexpr int kDT = D / 32;                       // 32-row M tiles of Oᵀ
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kOFloats = kDT * 16;                // O accumulator floats per lane
  static_assert(kOFloats * 64 * 4 <= kTileBytes, "a wave's O fits in one K buffer for the merge");
};

template <typename T, int D, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_keysplit_plain_kernel(KsParams p, const int* __restrict__ block_table,
                               const int* __restrict__ seq_lens) {
  using C = KpCfg<T, D>;
  using E = Elem<T>;
  using F = Frags<T>;
  using TT = Tile<C::kRowBytes>;
  typedef typename E::Frag Frag;
  constexpr int KS = C::kKS, MT = C::kMT, PS = C::kPS, DT = C::kDT;

  // K and V tiles of group g in buffer par: separate LDS objects, so that the
  // compiler sees that the tiles being loaded never alias the ones being read.
  __shared__ __attribute__((aligned(1024))) char k00[C::kTileBytes], k01[C::kTileBytes], k10[C::kTileBytes],
      k11[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v00[C::kTileBytes], v01[C::kTileBytes], v10[C::kTileBytes],
      v11[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char st_lds[2 * 2 * 64 * 4];  // merge: m, l of group 1's waves
  auto kbuf = [&](int g, int par) __attribute__((always_inline)) {
    return (lds_char*)(g ? (par ? k11 : k10) : (par ? k01 : k00));
  };
  auto vbuf = [&](int g, int par) __attribute__((always_inline)) {
    return (lds_char*)(g ? (par ? v11 : v10) : (par ? v01 : v00));
  };

  // Block -> (query tile, batch, head); causal: the heaviest tiles first.
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
  const int G = w >> 1, wl = w & 1;  // wave group, wave within the group
  const int h = lane >> 5, col = lane & 31;
  const int q0 = qt * C::kBR;
  const int qw = q0 + 32 * wl;       // first query row of this wave
  const int qrow = qw + col;         // this lane's query row
  const int diag = Nk - Nq;          // key j is visible to row i iff j <= i + diag (causal)

  const size_t q_row0 = (size_t)p.Hq * sr.tq + (size_t)hq * Nq;
  const size_t kv_row0 = (size_t)p.Hkv * sr.tk + (size_t)hkv * Nk;
  const size_t q_slab = q_row0 * D;
  const size_t kv_slab = kv_row0 * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + q_slab * 2, (uint32_t)Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.k + kv_slab * 2, (uint32_t)Nk * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)p.v + kv_slab * 2, (uint32_t)Nk * C::kRowBytes);

  int n_tiles = (Nk + C::kBC - 1) / C::kBC;
  if (CAUSAL) {
    const int last_key = min(q0 + C::kBR, Nq) - 1 + diag;
    n_tiles = last_key < 0 ? 0 : min(n_tiles, last_key / C::kBC + 1);
  }
  // Paged KV: the rows a wave moves of any tile lie in one 16-token page;
  // PageRef is that page for one tile (byte offset of its (page, kv head)
  // block in the cache and bytes of valid rows; 0 bytes reads zeros).
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
        const int pid = trow[t0 >> 4];
        if (pid >= 0 && pid < p.num_blocks) {  // a bad table entry reads as a page of zeros
          r.off = ((size_t)pid * p.Hkv + hkv) * (16 * C::kRowBytes);
          r.bytes = (uint32_t)min(16, Nk - (t0 & ~15)) * C::kRowBytes;
        }
      }
    }
    return r;
  };
  // K and V of tile j into buffers kd, vd (every wave moves its share).
  auto load_tile = [&](int j, lds_char* kd, lds_char* vd, const PageRef& pr) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      dma_tile<C::kRowBytes, C::kBC, C::kWaves, true>(make_rsrc((const char*)p.k + pr.off, pr.bytes), 0u, kd, w,
                                                      lane);
      dma_tile<C::kRowBytes, C::kBC, C::kWaves, true>(make_rsrc((const char*)p.v + pr.off, pr.bytes), 0u, vd, w,
                                                      lane);
    } else {
      dma_tile<C::kRowBytes, C::kBC, C::kWaves>(rk, (uint32_t)j * C::kBC * C::kRowBytes, kd, w, lane);
      dma_tile<C::kRowBytes, C::kBC, C::kWaves>(rv, (uint32_t)j * C::kBC * C::kRowBytes, vd, w, lane);
    }
  };
  // Pages of the two tiles (one per group) that the next step loads.
  PageRef pg_a = page_of(2), pg_b = page_of(3);
  if (n_tiles > 0) load_tile(0, kbuf(0, 0), vbuf(0, 0), page_of(0));
  if (n_tiles > 1) load_tile(1, kbuf(1, 0), vbuf(1, 0), page_of(1));

  // Qᵀ as the B operand of Sᵀ = K Qᵀ: lane holds row qrow, d = 16ks + 8h + 0..7.
  Frag qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    qf[ks] = F::template global_row<D>(rq, qrow, ks, h);
    if (p.neg_q) qf[ks] = E::negate(qf[ks]);
  }

  // Per-lane LDS offsets: fragment ks of K at kbase ^ 32 ks, column tile dt of
  // Vᵀ at vbase[u] ^ 64 dt (as in fwd_keysplit_kernel).
  uint32_t kbase = F::template row_off<TT>(sigma(col), 0, h);
  uint32_t vbase[2] = {F::template col_off<TT>(0, 0, lane), F::template col_off<TT>(0, 1, lane)};

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) o[dt] = f32x16{};
  f32x16 s[MT];   // scores of this wave's current tile
  Frag pf[PS];    // its probabilities
  float m = -INFINITY;  // running (possibly stale) max of scale*log2e*s, log2 domain
  float l = 0.f;        // this lane's share of the running sum
  const float c = p.c;  // > 0, so the max of c*s over a row is c*max(s)

  // Does this wave see any key of tile j?
  auto active = [&](int j) __attribute__((always_inline)) {
    return j < n_tiles && (!CAUSAL || j * C::kBC <= qw + 31 + diag);
  };

  auto gemm_s = [&](const lds_char* kb) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++) s[mt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const Frag a = F::lds_row_at(kb + 32 * mt * C::kRowBytes, kbase ^ (uint32_t)(32 * ks));
        s[mt] = E::mma(a, qf[ks], s[mt]);
      }
    sched_units<KS * MT, 1, 1, 2>();
  };
  auto gemm_pv = [&](const lds_char* vb) __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < PS; ps++)
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        const Frag a = F::lds_col_at(vb + 16 * ps * C::kRowBytes, vbase[0] ^ (uint32_t)(64 * dt),
                                     vbase[1] ^ (uint32_t)(64 * dt));
        o[dt] = E::mma(a, pf[ps], o[dt]);
      }
    sched_units<PS * DT, 2, 1, 2>();
  };
  // Register r of M tile mt holds key k0 + 32*mt + 16*(r/8) + 8h + (r%8).
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * C::kBC;
    if ((k0 + C::kBC > Nk) || (CAUSAL && k0 + C::kBC - 1 > qw + diag)) {
      const int horizon = CAUSAL ? min(qrow + diag, Nk - 1) : Nk - 1;
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int key = k0 + 32 * mt + 16 * (r >> 3) + 8 * h + (r & 7);
          if (key > horizon) s[mt][r] = -INFINITY;
        }
    }
    float x[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int r = (mt == 0 ? 4 : 0); r < 16; r += 8)
#pragma unroll
        for (int i = 0; i < 4; i++)
          x[i] = r + 4 + i < 16 ? vmax(vmax(x[i], s[mt][r + i]), s[mt][r + 4 + i]) : vmax(x[i], s[mt][r + i]);
    const float mx = max_halves(vmax(vmax(x[0], x[1]), vmax(x[2], x[3]))) * c;
    // Move the running max only if it grows by more than kTau.
    const bool grow = mx > m + kTau;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m - mx) : 1.f;
      m = grow ? mx : m;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; dt++) o[dt] *= alpha;
    }
    const float m_use = m == -INFINITY ? 0.f : m;  // rows that have seen no key yet
    float rs[4];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        s[mt][r] = fast_exp2(fmaf(s[mt][r], c, -m_use));
        rs[r & 3] = (mt == 0 && r < 4) ? s[mt][r] : rs[r & 3] + s[mt][r];
      }
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    // Pᵀ k block ps = registers 8*(ps%2).. of M tile ps/2.
#pragma unroll
    for (int ps = 0; ps < PS; ps++) {
      float pv[8];
#pragma unroll
      for (int t = 0; t < 8; t++) pv[t] = s[ps >> 1][8 * (ps & 1) + t];
      pf[ps] = E::pack(pv);
    }
  };

  // ---- step u (one barrier after each): both groups' tiles of step u + 1
  // (tiles 2u + 2, 2u + 3) are loaded into the other buffers, then each wave
  // runs S, softmax and PV of its group's tile 2u + g.  Steps are unrolled by
  // two and each group runs its own copy of the loop, so every buffer is a
  // compile-time object.
  const int n_steps = (n_tiles + 1) >> 1;
  auto step = [&](auto gc, auto pc, int u) __attribute__((always_inline)) {
    constexpr int g = decltype(gc)::value;    // this wave's group
    constexpr int par = decltype(pc)::value;  // parity of u
    // The lane offsets are re-hidden from the compiler at every step, so
    // that it adds them to the buffer bases inside the step instead of
    // keeping one hoisted address register per (buffer, fragment) pair.
    asm volatile("" : "+v"(kbase), "+v"(vbase[0]), "+v"(vbase[1]));
    if (2 * u + 2 < n_tiles) load_tile(2 * u + 2, kbuf(0, par ^ 1), vbuf(0, par ^ 1), pg_a);
    if (2 * u + 3 < n_tiles) load_tile(2 * u + 3, kbuf(1, par ^ 1), vbuf(1, par ^ 1), pg_b);
    const int j = 2 * u + g;
    if (active(j)) {
      gemm_s(kbuf(g, par));
      softmax(j);
      gemm_pv(vbuf(g, par));
    }
    if constexpr (PAGED) {
      // Table entries of the next step's tiles, read after this step's LDS
      // work (the empty asm keeps them there) so that their wait merges with
      // the barrier's.
      asm volatile("" ::: "memory");
      pg_a = page_of(2 * u + 4);
      pg_b = page_of(2 * u + 5);
    }
    wait_vmem();
    barrier_lds();
  };
  wait_vmem();
  barrier_lds();
  auto run = [&](auto gc) __attribute__((always_inline)) {
    for (int u = 0; u < n_steps; u += 2) {
      step(gc, Int<0>{}, u);
      if (u + 1 < n_steps) step(gc, Int<1>{}, u + 1);
    }
  };
  if (G == 0) run(Int<0>{});
  else run(Int<1>{});

  // ---- merge: group 1 hands (O, m, l) to the group-0 wave with its rows
  // through its own K buffers (free once the last step's barrier has passed);
  // that wave rescales both parts to the common max and adds them.
  lds_char* const mg = wl ? kbuf(1, 1) : kbuf(1, 0);
  __attribute__((address_space(3))) float* const st =
      (__attribute__((address_space(3))) float*)((lds_char*)st_lds + wl * 2 * 64 * 4);
  if (G == 1) {
    st[lane] = m;
    st[64 + lane] = l;
#pragma unroll
    for (int f4 = 0; f4 < C::kOFloats / 4; f4++) {
      const int dt = f4 / 4, r = 4 * (f4 % 4);
      *(__attribute__((address_space(3))) f32x4*)(mg + (f4 * 64 + lane) * 16) =
          f32x4{o[dt][r], o[dt][r + 1], o[dt][r + 2], o[dt][r + 3]};
    }
  }
  barrier_lds();
  if (G == 1) return;
  {
    const float m1 = st[lane], l1 = st[64 + lane];
    const float M = vmax(m, m1);
    const float a0 = m == -INFINITY ? 0.f : fast_exp2(m - M);
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - M);
    l = a0 * l + a1 * l1;
    m = M;
#pragma unroll
    for (int f4 = 0; f4 < C::kOFloats / 4; f4++) {
      const int dt = f4 / 4, r = 4 * (f4 % 4);
      const f32x4 v4 = *(__attribute__((address_space(3))) f32x4*)(mg + (f4 * 64 + lane) * 16);
#pragma unroll
      for (int i = 0; i < 4; i++) o[dt][r + i] = fmaf(a1, v4[i], a0 * o[dt][r + i]);
    }
  }

  // ---- epilogue (group 0): O = Oᵀ / l, LSE = m + log2(l) in natural log.
  const float lt = sum_halves(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc((char*)p.o + q_slab * 2, (uint32_t)Nq * C::kRowBytes);
#pragma unroll
  for (int dt = 0; dt < DT; dt++)
#pragma unroll
    for (int a4 = 0; a4 < 4; a4++) {
      const int d0 = 32 * dt + 8 * a4 + 4 * h;
      F::store4(ro, (uint32_t)qrow * C::kRowBytes + d0 * 2, o[dt][4 * a4] * inv, o[dt][4 * a4 + 1] * inv,
                o[dt][4 * a4 + 2] * inv, o[dt][4 * a4 + 3] * inv);
    }
  if (h == 0) {
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + q_row0, (uint32_t)Nq * 4);
    const float lse = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
    buf_store4(rl, (uint32_t)qrow * 4, __builtin_bit_cast(uint32_t, lse));
  }
}

template <typename T, int D, bool CAUSAL, bool PAGED>
hipError_t launch_typed(const FwdArgs& a, hipStream_t stream) {
  using C = KsCfg<T, D>;
  KsParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.lse = a.lse;
  p.cu_q = a.cu_q; p.cu_k = a.cu_k;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.tot_q = a.tot_q; p.tot_k = a.tot_k;
  p.max_blocks = a.max_blocks; p.num_blocks = a.num_blocks;
  const ExpScale es = exp_scale(a.scale * kLog2e);
  p.c = es.c; p.neg_q = es.neg_q;
  // Causal grids with head sizes up to 64 run the 4-wave kernel: its 64-row
  // work-groups, two per compute unit, spread the heavy diagonal-end tiles
  // over more compute units (mha_f16: 13.2 against 15.5 us).  Non-causal
  // grids keep the 8-wave slot schedule, whose alternation has the higher
  // throughput when every work-group carries the same load (15.3 against 16.1).
  if constexpr (D <= 64 && CAUSAL) {
    using P = KpCfg<T, D>;
    const unsigned grid = (unsigned)((a.Nq + P::kBR - 1) / P::kBR) * a.B * a.Hq;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_keysplit_plain_kernel<T, D, CAUSAL, PAGED>), dim3(grid), dim3(64 * P::kWaves), 0,
                       stream, p, a.block_table, a.seq_lens);
  } else {
    const unsigned grid = (unsigned)((a.Nq + C::kBR - 1) / C::kBR) * a.B * a.Hq;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_keysplit_kernel<T, D, CAUSAL, PAGED>), dim3(grid), dim3(64 * C::kWaves), 0, stream, p,
                       a.block_table, a.seq_lens);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mask(const FwdArgs& a, hipStream_t s) {
  if (a.block_table)
    return a.causal ? launch_typed<T, D, true, true>(a, s) : launch_typed<T, D, false, true>(a, s);
  return a.causal ? launch_typed<T, D, true, false>(a, s) : launch_typed<T, D, false, false>(a, s);
}

template <typename T>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  switch (a.d) {
    case 32: return launch_mask<T, 32>(a, s);
    case 64: return launch_mask<T, 64>(a, s);
    case 128: return launch_mask<T, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_keysplit(const FwdArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 1: return launch_d<_Float16>(a, stream);
    case 2: return launch_d<__bf16>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
