// fa_bwd.hip -- exact attention backward for gfx950 (recomputation).
//
// The tutorial "FlashAttention and efficient attention kernels" (sections
// "Backward" and "Backward recompute flow") and the concept page
// "Flash-Attention" ("Core idea": recomputation instead of stored softmax
// intermediates) fix the flow: reload Q, K, V blocks and the saved per-row
// statistics, rebuild S and P on chip, combine with dO into dQ, dK, dV, and
// drop every block once used.  The pages print no gradient formula; the
// kernels evaluate the chain rule of the three-step definition:
//   P  = exp(scale*S - LSE)          (no running max needed: LSE is final)
//   dV = Pᵀ dO,   dP = dO Vᵀ,   dS = P ∘ (dP - D),   D_i = Σ_c dO_ic O_ic
//   dQ = scale dS K,   dK = scale dSᵀ Q
//
// Three kernels, all deterministic (no atomics):
//   bwd_prep : -D_i and LSE_i*log2(e) per query row (a streaming pass; D is
//              kept negated so that the dK/dV kernel can start its dP
//              accumulators from it and get dP - D out of the products);
//   bwd_dkdv : KV-outer.  A work-group keeps 128 keys (32 per wave) and their
//              K, V rows in registers and walks every query tile (of every
//              query head of its group) that can see them.  S = Q Kᵀ is
//              computed with queries as the A rows and keys as lanes, so P
//              and dS come out in exactly the B-operand layout of dVᵀ += dOᵀ P
//              and dKᵀ += Qᵀ dS; Qᵀ and dOᵀ come from transposing LDS reads.
//   bwd_dq   : Q-outer, shaped like the forward: Sᵀ = K Qᵀ and dPᵀ = V dOᵀ
//              with queries as lanes, then dQᵀ += Kᵀ dSᵀ.
// P and dS are rounded to the input type before their products (float32
// inputs keep float32).
#include "fa_device.hpp"
#include "fa_kernels.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// Preprocess
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                       const float* __restrict__ lse, float* __restrict__ dsum,
                                                       float* __restrict__ lse2, int64_t rows) {
  constexpr int kES = (int)sizeof(T);
  constexpr int kEPC = 16 / kES;  // elements per 16-byte chunk
  constexpr int kTPR = D / kEPC;  // threads per row (4..32)
  typedef T tv __attribute__((ext_vector_type(kEPC)));
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / kTPR;
  const int c = (int)(gid % kTPR);
  float acc = 0.f;
  if (row < rows) {
    const tv a = __builtin_bit_cast(tv, *(const u32x4*)(o + row * D + c * kEPC));
    const tv b = __builtin_bit_cast(tv, *(const u32x4*)(dout + row * D + c * kEPC));
#pragma unroll
    for (int i = 0; i < kEPC; i++) acc = fmaf((float)a[i], (float)b[i], acc);
  }
#pragma unroll
  for (int off = kTPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && c == 0) {
    dsum[row] = -acc;  // stored negated: the kernels add it (or start dP's accumulator from it)
    const float L = lse[row];
    // Rows that see no key carry LSE = -inf; +inf makes exp2(s - lse2) vanish.
    lse2[row] = L == -INFINITY ? INFINITY : L * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV (KV-outer)
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkvCfg {
  static constexpr int kWaves = 4;
  static constexpr int kBKV = 32 * kWaves;  // keys per work-group
  static constexpr int kES = Elem<T>::kBytes;
  static constexpr int kRowBytes = D * kES;
  static constexpr int kBQ = 64;            // query rows per step
  static constexpr int kKS = D / 16;
  static constexpr int kMT = kBQ / 32;      // 32-query M tiles of S
  static constexpr int kPS = kBQ / 16;      // 16-query k blocks of dVᵀ/dKᵀ
  static constexpr int kDT = D / 32;
  static constexpr int kTileBytes = kBQ * kRowBytes;
  static constexpr int kStatBytes = 2 * kBQ * 4;  // lse2, dsum of the step's rows
  static_assert(kStatBytes == 512, "stats are staged by 32 lanes x 16 B");
};

struct DkvParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse2;
  const float* dsum;
  void* dk;
  void* dv;
  const int* cu_q;  // packed batch: cumulative query / key counts [B + 1], else null
  const int* cu_k;
  int B, Hq, Hkv, Nq, Nk;  // Nq, Nk: the lengths (dense) or their bounds (packed)
  int tot_q, tot_k;        // packed batch: total query / key tokens
  float c;      // scale * log2(e)
  float scale;
  // The same exponent scale for the 16-bit kernel, which flips K's sign for
  // a negative scale: |c| (2^-100 for a zero scale) and the flip.
  float c_mag;
  int neg_k;
};

// Eight consecutive floats of the LDS stats area starting at float index i.
__device__ __forceinline__ void lds_read8f(const lds_char* base, int i, float* out) {
  const u32x4 a = lds_read16(base, (uint32_t)i * 4), b = lds_read16(base, (uint32_t)i * 4 + 16);
#pragma unroll
  for (int j = 0; j < 4; j++) { out[j] = as_float(a[j]); out[4 + j] = as_float(b[j]); }
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(DkvParams p) {
  using C = DkvCfg<T, D>;
  using E = Elem<T>;
  using F = Frags<T>;
  using TT = Tile<C::kRowBytes>;
  typedef typename E::Frag Frag;

  // Double-buffered Q, dO and stats tiles, each buffer its own LDS object: the
  // compiler then knows that the tiles being loaded never alias the tiles
  // being read, and does not make the reads wait for the loads.
  __shared__ __attribute__((aligned(1024))) char q_lds0[C::kTileBytes], q_lds1[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char do_lds0[C::kTileBytes], do_lds1[C::kTileBytes];
  __shared__ __attribute__((aligned(512))) char st_lds0[C::kStatBytes], st_lds1[C::kStatBytes];
  auto qbuf = [&](int par) __attribute__((always_inline)) { return (lds_char*)(par ? q_lds1 : q_lds0); };
  auto dobuf = [&](int par) __attribute__((always_inline)) { return (lds_char*)(par ? do_lds1 : do_lds0); };
  auto stbuf = [&](int par) __attribute__((always_inline)) { return (lds_char*)(par ? st_lds1 : st_lds0); };

  // Block -> (key tile, batch, kv head).  Under the causal mask the first key
  // tiles are seen by the most query rows, so they go first.
  const int bh_count = p.B * p.Hkv;
  const int id = blockIdx.x;
  const int bhk = id % bh_count;
  const int kt = id / bh_count;
  const int b = bhk / p.Hkv, hkv = bhk - b * p.Hkv;
  const int g = p.Hq / p.Hkv;
  // The grid covers the longest sequence; blocks past a shorter one's keys leave at once.
  const SeqRows sr = seq_rows(p.cu_q, p.cu_k, b, p.Nq, p.Nk, p.tot_q, p.tot_k);
  const int Nq = sr.nq, Nk = sr.nk;
  if (kt * C::kBKV >= Nk) return;
  const size_t kv_row0 = (size_t)p.Hkv * sr.tk + (size_t)hkv * Nk;  // first row of this (sequence, kv head)
  // First row of query head hq of this sequence (in Q, dO and the row terms).
  auto q_row0 = [&](int hq) __attribute__((always_inline)) { return (size_t)p.Hq * sr.tq + (size_t)hq * Nq; };

  const int lane = lane_id(), w = wave_id();
  const int h = lane >> 5, col = lane & 31;
  const int k0 = kt * C::kBKV;
  const int kw = k0 + 32 * w;   // first key of this wave
  const int key = kw + col;     // this lane's key
  const int diag = Nk - Nq; // key j is visible to row i iff j <= i + diag (causal)

  const size_t kv_slab = kv_row0 * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.k + kv_slab * C::kES, (uint32_t)Nk * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)p.v + kv_slab * C::kES, (uint32_t)Nk * C::kRowBytes);

  // Query tiles that can see this work-group's keys, for each head of the group.
  const int n_qt = (Nq + C::kBQ - 1) / C::kBQ;
  const int qt0 = CAUSAL ? max(0, k0 - diag) / C::kBQ : 0;
  const int per_head = n_qt - qt0;
  const int steps = g * per_head;

  auto load_step = [&](int s, int buf) __attribute__((always_inline)) {
    const int hq = hkv * g + s / per_head;
    const int qt = qt0 + s % per_head;
    const size_t qr0 = q_row0(hq);
    const size_t q_slab = qr0 * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + q_slab * C::kES, (uint32_t)Nq * C::kRowBytes);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const char*)p.dout + q_slab * C::kES, (uint32_t)Nq * C::kRowBytes);
    const uint32_t g0 = (uint32_t)qt * C::kBQ * C::kRowBytes;
    dma_tile<C::kRowBytes, C::kBQ, C::kWaves>(rq, g0, buf ? qbuf(1) : qbuf(0), w, lane);
    dma_tile<C::kRowBytes, C::kBQ, C::kWaves>(rdo, g0, buf ? dobuf(1) : dobuf(0), w, lane);
    // Per-row stats of the step: lanes 0-15 stage lse2, lanes 16-31 dsum.
    if (w == 0) {
      const uint32_t off = (uint32_t)qt * C::kBQ * 4 + (lane & 15) * 16;
      lds_char* st = buf ? stbuf(1) : stbuf(0);
      if (lane < 16) buf_load16_to_lds(make_rsrc(p.lse2 + qr0, (uint32_t)Nq * 4), off, st);
      else if (lane < 32) buf_load16_to_lds(make_rsrc(p.dsum + qr0, (uint32_t)Nq * 4), off, st);
    }
  };

  if (steps > 0) load_step(0, 0);

  // Kᵀ and Vᵀ as B operands (k = d, column = this lane's key).
  Frag kf[C::kKS], vf[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ks++) {
    kf[ks] = F::template global_row<D>(rk, key, ks, h);
    vf[ks] = F::template global_row<D>(rv, key, ks, h);
  }
  f32x16 dk[C::kDT], dv[C::kDT];
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++) { dk[dt] = f32x16{}; dv[dt] = f32x16{}; }

  // Per-lane LDS offsets of the Q / dO row fragments (A rows are sigma-permuted
  // queries) and of the Qᵀ / dOᵀ column fragments.
  uint32_t roff[C::kKS], coff[C::kDT][2];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ks++) roff[ks] = F::template row_off<TT>(sigma(col), ks, h);
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++)
#pragma unroll
    for (int u = 0; u < 2; u++) coff[dt][u] = F::template col_off<TT>(32 * dt, u, lane);

  wait_vmem();
  barrier_lds();

  // One step: query rows i0 .. i0 + kBQ - 1 of one query head.
  auto step = [&](int s, const lds_char* qb, const lds_char* dob, const lds_char* stb) __attribute__((always_inline)) {
    const int i0 = (qt0 + s % per_head) * C::kBQ;  // first query row of the step
    if (CAUSAL && i0 + C::kBQ - 1 + diag < kw) return;
    // ---- S = Q Kᵀ and dP = dO Vᵀ; A rows are sigma-permuted queries.
    f32x16 sv[C::kMT], dp[C::kMT];
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++) { sv[mt] = f32x16{}; dp[mt] = f32x16{}; }
#pragma unroll
    for (int ks = 0; ks < C::kKS; ks++) {
#pragma unroll
      for (int mt = 0; mt < C::kMT; mt++) {
        if constexpr (C::kES == 2) {
          sv[mt] = E::mma(F::lds_row_at(qb + 32 * mt * C::kRowBytes, roff[ks]), kf[ks], sv[mt]);
          dp[mt] = E::mma(F::lds_row_at(dob + 32 * mt * C::kRowBytes, roff[ks]), vf[ks], dp[mt]);
        } else {
          const int row = 32 * mt + sigma(col);
          sv[mt] = E::mma(F::template lds_row<TT>(qb, row, ks, h), kf[ks], sv[mt]);
          dp[mt] = E::mma(F::template lds_row<TT>(dob, row, ks, h), vf[ks], dp[mt]);
        }
      }
    }
    if constexpr (C::kES == 2) sched_reads_ahead<2 * C::kKS * C::kMT, 2 * C::kKS * C::kMT, 4>();
    // ---- P and dS.  Register r of M tile mt holds query
    //      i0 + 32*mt + 16*(r/8) + 8h + (r%8) for this lane's key.
    //      Only steps that cross the causal diagonal mask P (a uniform branch).
    float dd[C::kMT][2][8];
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
      for (int u = 0; u < 2; u++) {
        float l2[8];
        lds_read8f(stb, 32 * mt + 16 * u + 8 * h, l2);
        lds_read8f(stb, C::kBQ + 32 * mt + 16 * u + 8 * h, dd[mt][u]);
#pragma unroll
        for (int t = 0; t < 8; t++) sv[mt][8 * u + t] = fast_exp2(fmaf(sv[mt][8 * u + t], p.c, -l2[t]));
      }
    if (CAUSAL && kw + 31 > i0 + diag) {
#pragma unroll
      for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
        for (int r = 0; r < 16; r++)
          if (key > i0 + 32 * mt + 16 * (r >> 3) + 8 * h + (r & 7) + diag) sv[mt][r] = 0.f;
    }
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) dp[mt][r] = sv[mt][r] * (dp[mt][r] + dd[mt][r >> 3][r & 7]);  // dd = -D
    // ---- dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS (column = key, k = query).
#pragma unroll
    for (int ps = 0; ps < C::kPS; ps++) {
      float pv[8], dsv[8];
#pragma unroll
      for (int t = 0; t < 8; t++) { pv[t] = sv[ps >> 1][8 * (ps & 1) + t]; dsv[t] = dp[ps >> 1][8 * (ps & 1) + t]; }
      const Frag pf = E::pack(pv), dsf = E::pack(dsv);
#pragma unroll
      for (int dt = 0; dt < C::kDT; dt++) {
        if constexpr (C::kES == 2) {
          dv[dt] = E::mma(F::lds_col_at(dob + 16 * ps * C::kRowBytes, coff[dt][0], coff[dt][1]), pf, dv[dt]);
          dk[dt] = E::mma(F::lds_col_at(qb + 16 * ps * C::kRowBytes, coff[dt][0], coff[dt][1]), dsf, dk[dt]);
        } else {
          dv[dt] = E::mma(F::template lds_col<TT>(dob, 16 * ps, 32 * dt, lane), pf, dv[dt]);
          dk[dt] = E::mma(F::template lds_col<TT>(qb, 16 * ps, 32 * dt, lane), dsf, dk[dt]);
        }
      }
    }
    if constexpr (C::kES == 2) sched_reads_ahead<4 * C::kPS * C::kDT, 2 * C::kPS * C::kDT, 4>();
  };

  if constexpr (C::kES == 2) {
    // Two steps per trip so that every buffer is a compile-time LDS object.
    for (int s = 0; s < steps; s += 2) {
      if (s + 1 < steps) load_step(s + 1, 1);
      step(s, qbuf(0), dobuf(0), stbuf(0));
      wait_vmem();
      barrier_lds();
      if (s + 1 < steps) {
        if (s + 2 < steps) load_step(s + 2, 0);
        step(s + 1, qbuf(1), dobuf(1), stbuf(1));
        wait_vmem();
        barrier_lds();
      }
    }
  } else {
    // float32: one step per trip (its larger fragments leave no room to unroll).
    for (int s = 0; s < steps; s++) {
      const int buf = s & 1;
      if (s + 1 < steps) load_step(s + 1, buf ^ 1);
      step(s, qbuf(buf), dobuf(buf), stbuf(buf));
      wait_vmem();
      barrier_lds();
    }
  }

  // ---- epilogue: dK = scale * dKᵀ acc, dV; lane's column is its key.
  const __amdgpu_buffer_rsrc_t wk = make_rsrc((char*)p.dk + kv_slab * C::kES, (uint32_t)Nk * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t wv = make_rsrc((char*)p.dv + kv_slab * C::kES, (uint32_t)Nk * C::kRowBytes);
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++)
#pragma unroll
    for (int a4 = 0; a4 < 4; a4++) {
      const uint32_t off = (uint32_t)key * C::kRowBytes + (32 * dt + 8 * a4 + 4 * h) * C::kES;
      F::store4(wk, off, dk[dt][4 * a4] * p.scale, dk[dt][4 * a4 + 1] * p.scale, dk[dt][4 * a4 + 2] * p.scale,
                dk[dt][4 * a4 + 3] * p.scale);
      F::store4(wv, off, dv[dt][4 * a4], dv[dt][4 * a4 + 1], dv[dt][4 * a4 + 2], dv[dt][4 * a4 + 3]);
    }
}

// dK, dV for 16-bit types, software-pipelined.  One wave per SIMD owns 32
// keys (as above).  Step i of the main loop overlaps, within each wave,
//   P(i), dS(i) on the VALU   with   dVᵀ, dKᵀ += ... of step i-1  and
//                                    S, dP of step i+1 on the matrix core.
// The products run in chunks of four, fenced from each other, and the P/dS
// work is cut into stages that follow a fixed chunk schedule (see fused).
// Steps rotate through four LDS buffers: step i+2 is loaded at the top of
// step i into the buffer of step i-2, after a barrier that both publishes
// step i+1's tiles and frees that buffer.
// Under the causal mask the query tiles that cross the diagonal (at most the
// first three of each head) are done first, one at a time with a masked step;
// the pipelined steps then mask nothing.  Masked scores are set to -inf
// before the exponential; a negative scale flips the sign of K instead, a
// zero scale becomes a tiny positive one, so P is 0 there with no NaN.  The
// first pipelined step multiplies P/dS by a zeroed buffer, so it adds nothing.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv16_kernel(DkvParams p) {
  using C = DkvCfg<T, D>;
  using E = Elem<T>;
  using F = Frags<T>;
  using TT = Tile<C::kRowBytes>;
  typedef typename E::Frag Frag;
  constexpr int KS = C::kKS, MT = C::kMT, PS = C::kPS, DT = C::kDT;

  __shared__ __attribute__((aligned(1024))) char q_l0[C::kTileBytes], q_l1[C::kTileBytes], q_l2[C::kTileBytes],
      q_l3[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char do_l0[C::kTileBytes], do_l1[C::kTileBytes], do_l2[C::kTileBytes],
      do_l3[C::kTileBytes];
  // Row statistics of a step: lse2 in the first 256 bytes, dsum in the next;
  // every wave owns one 256-byte slot that its stats load writes.
  constexpr int kStatArea = 256 * C::kWaves;
  static_assert(C::kBQ * 4 == 256, "a step's rows fill one slot");
  __shared__ __attribute__((aligned(1024))) char st_l0[kStatArea], st_l1[kStatArea], st_l2[kStatArea],
      st_l3[kStatArea];
  auto qbuf = [&](int i) __attribute__((always_inline)) {
    return (lds_char*)(i == 0 ? q_l0 : i == 1 ? q_l1 : i == 2 ? q_l2 : q_l3);
  };
  auto dobuf = [&](int i) __attribute__((always_inline)) {
    return (lds_char*)(i == 0 ? do_l0 : i == 1 ? do_l1 : i == 2 ? do_l2 : do_l3);
  };
  auto stbuf = [&](int i) __attribute__((always_inline)) {
    return (lds_char*)(i == 0 ? st_l0 : i == 1 ? st_l1 : i == 2 ? st_l2 : st_l3);
  };

  const int bh_count = p.B * p.Hkv;
  const int id = blockIdx.x;
  const int bhk = id % bh_count;
  const int kt = id / bh_count;
  const int b = bhk / p.Hkv, hkv = bhk - b * p.Hkv;
  const int g = p.Hq / p.Hkv;
  // The grid covers the longest sequence; blocks past a shorter one's keys leave at once.
  const SeqRows sr = seq_rows(p.cu_q, p.cu_k, b, p.Nq, p.Nk, p.tot_q, p.tot_k);
  const int Nq = sr.nq, Nk = sr.nk;
  if (kt * C::kBKV >= Nk) return;
  const size_t kv_row0 = (size_t)p.Hkv * sr.tk + (size_t)hkv * Nk;  // first row of this (sequence, kv head)
  // First row of query head hq of this sequence (in Q, dO and the row terms).
  auto q_row0 = [&](int hq) __attribute__((always_inline)) { return (size_t)p.Hq * sr.tq + (size_t)hq * Nq; };

  const int lane = lane_id(), w = wave_id();
  const int h = lane >> 5, col = lane & 31;
  const int k0 = kt * C::kBKV;
  const int kw = k0 + 32 * w;
  const int key = kw + col;
  const int diag = Nk - Nq;
  const bool neg = p.neg_k;
  const float c = p.c_mag;

  const size_t kv_slab = kv_row0 * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.k + kv_slab * 2, (uint32_t)Nk * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)p.v + kv_slab * 2, (uint32_t)Nk * C::kRowBytes);

  // Query tiles per head that see this work-group's keys: the first n_diag
  // of them cross the causal diagonal (every later row sees all 128 keys),
  // the other n_rest form the pipelined steps, head after head.
  const int n_qt = (Nq + C::kBQ - 1) / C::kBQ;
  const int qt0 = CAUSAL ? max(0, k0 - diag) / C::kBQ : 0;
  const int per_head = n_qt - qt0;
  const int n_diag = CAUSAL ? max(0, min(per_head, (k0 + C::kBKV - 2 - diag) / C::kBQ - qt0 + 1)) : 0;
  const int n_rest = per_head - n_diag;
  const int n_dsteps = g * n_diag;
  const int steps = g * n_rest;

  // Loads of query tile qt of head hh of the group into buffer buf.  An
  // invalid tile issues the same instructions on empty ranges, which read
  // nothing, so that no wave branches.
  auto load_tile = [&](int hh, int qt, int buf, bool valid) __attribute__((always_inline)) {
    const size_t qr0 = q_row0(hkv * g + hh);
    const size_t q_slab = qr0 * D;
    const uint32_t bytes = valid ? (uint32_t)Nq * C::kRowBytes : 0u;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + q_slab * 2, bytes);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const char*)p.dout + q_slab * 2, bytes);
    const uint32_t g0 = (uint32_t)qt * C::kBQ * C::kRowBytes;
    dma_tile<C::kRowBytes, C::kBQ, C::kWaves>(rq, g0, qbuf(buf), w, lane);
    dma_tile<C::kRowBytes, C::kBQ, C::kWaves>(rdo, g0, dobuf(buf), w, lane);
    // Row statistics, one dword per lane: wave 0 stages lse2 and wave 1
    // dsum; waves 2 and 3 load from an empty range into their own slots.
    const float* src = (w == 0 ? p.lse2 : p.dsum) + qr0;
    const uint32_t nb = (valid && w < 2) ? (uint32_t)Nq * 4 : 0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(src, nb), (lds_void*)(stbuf(buf) + w * 256), 4,
                                             (uint32_t)qt * C::kBQ * 4 + lane * 4, 0, 0, 0);
  };
  // (An invalid step maps to tile 0 of head 0; the divisors are kept
  // nonzero for the calls that load nothing.)
  const int n_rest_d = max(n_rest, 1), n_diag_d = max(n_diag, 1);
  auto load_step = [&](int s, int buf, bool valid) __attribute__((always_inline)) {
    s = valid ? s : 0;
    load_tile(s / n_rest_d, qt0 + n_diag + s % n_rest_d, buf, valid);
  };
  auto load_diag = [&](int s, int buf, bool valid) __attribute__((always_inline)) {
    s = valid ? s : 0;
    load_tile(s / n_diag_d, qt0 + s % n_diag_d, buf, valid);
  };

  // Kᵀ and Vᵀ as B operands (k = d, column = this lane's key), loaded before
  // the first tiles: the first step then waits for these and its own tile
  // only, while the two pipelined steps' tiles are still in flight.
  Frag kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    kf[ks] = F::template global_row<D>(rk, key, ks, h);
    vf[ks] = F::template global_row<D>(rv, key, ks, h);
  }
  // The first three tiles' loads are issued whether or not their tiles exist
  // (an absent one reads an empty range), so that every wave has the same
  // fixed number of loads in flight behind the K/V fragments.
  __builtin_amdgcn_sched_barrier(0);
  load_diag(0, 2, n_dsteps > 0);
  load_step(0, 0, steps > 0);
  load_step(1, 1, steps > 1);
  __builtin_amdgcn_sched_barrier(0);
  // Vector-memory instructions of one tile load (per wave): Q, dO, stats.
  using TS = DmaShape<C::kRowBytes, C::kBQ, C::kWaves>;
  static_assert(TS::kActive == C::kWaves, "every wave issues the same tile loads");
  constexpr int kTileLoads = 2 * TS::kPer + 1;
#pragma unroll
  for (int ks = 0; ks < KS; ks++)
    if (neg) kf[ks] = E::negate(kf[ks]);
  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) { dk[dt] = f32x16{}; dv[dt] = f32x16{}; }
  // Per-lane LDS offsets: Q / dO row fragments (A rows are sigma-permuted
  // queries), Qᵀ / dOᵀ column fragments, and this lane's rows of a stats area.
  uint32_t roff[KS], coff[DT][2];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) roff[ks] = F::template row_off<TT>(sigma(col), ks, h);
#pragma unroll
  for (int dt = 0; dt < DT; dt++)
#pragma unroll
    for (int u = 0; u < 2; u++) coff[dt][u] = F::template col_off<TT>(32 * dt, u, lane);
  uint32_t soff = 32 * h;

  f32x16 sv[MT], dp[MT];
  Frag pa[PS], da[PS], pb[PS], db[PS];  // P and dS fragments of two consecutive steps
#pragma unroll
  for (int ps = 0; ps < PS; ps++) { pa[ps] = Frag{}; da[ps] = Frag{}; pb[ps] = Frag{}; db[ps] = Frag{}; }

  // -D of the rows of M tile mt of a step, in the layout of its dP
  // accumulator (register r: query 32*mt + 16*(r/8) + 8h + (r%8)).
  auto neg_d = [&](const lds_char* stb, int mt) __attribute__((always_inline)) {
    float lo[8], hi[8];
    lds_read8f(stb, C::kBQ + 32 * mt + 8 * h, lo);
    lds_read8f(stb, C::kBQ + 32 * mt + 16 + 8 * h, hi);
    f32x16 r;
#pragma unroll
    for (int t = 0; t < 8; t++) { r[t] = lo[t]; r[8 + t] = hi[t]; }
    return r;
  };
  // S = Q Kᵀ and dP = dO Vᵀ of one step (A rows: sigma-permuted queries).
  // With NEG the dP accumulators start from -D, so that they end as dP - D.
  auto gemm_sdp = [&](const lds_char* qb, const lds_char* dob, const lds_char* stb, auto negc)
      __attribute__((always_inline)) {
    constexpr bool NEG = decltype(negc)::value;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      sv[mt] = f32x16{};
      if constexpr (NEG) dp[mt] = neg_d(stb, mt);
      else dp[mt] = f32x16{};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        sv[mt] = E::mma(F::lds_row_at(qb + 32 * mt * C::kRowBytes, roff[ks]), kf[ks], sv[mt]);
        dp[mt] = E::mma(F::lds_row_at(dob + 32 * mt * C::kRowBytes, roff[ks]), vf[ks], dp[mt]);
      }
  };
  // Register r of M tile mt holds query i0 + 32*mt + 16*(r/8) + 8h + (r%8).
  auto mask = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        if (key > i0 + 32 * mt + 16 * (r >> 3) + 8 * h + (r & 7) + diag) sv[mt][r] = -INFINITY;
  };
  // P = exp2(c s - lse2), dS = P (dP - D), both rounded to T as B operands.
  auto p_ds = [&](const lds_char* stb, Frag (&pn)[PS], Frag (&dn)[PS]) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int u = 0; u < 2; u++) {
        float l2[8], pv[8], dsv[8];
        lds_read8f(stb, 32 * mt + 16 * u + 8 * h, l2);
#pragma unroll
        for (int t = 0; t < 8; t++) {
          pv[t] = fast_exp2(fmaf(sv[mt][8 * u + t], c, -l2[t]));
          dsv[t] = pv[t] * dp[mt][8 * u + t];
        }
        pn[2 * mt + u] = E::pack(pv);
        dn[2 * mt + u] = E::pack(dsv);
      }
  };
  // dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS of one step (column = key, k = query).
  auto gemm_dvdk = [&](const lds_char* qb, const lds_char* dob, const Frag (&pf)[PS], const Frag (&dsf)[PS])
      __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < PS; ps++)
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        dv[dt] = E::mma(F::lds_col_at(dob + 16 * ps * C::kRowBytes, coff[dt][0], coff[dt][1]), pf[ps], dv[dt]);
        dk[dt] = E::mma(F::lds_col_at(qb + 16 * ps * C::kRowBytes, coff[dt][0], coff[dt][1]), dsf[ps], dk[dt]);
      }
  };

  // ---- Diagonal tiles (causal only), unpipelined, alternating between
  // buffers 2 and 3; each step's barrier publishes its tiles and frees the
  // other buffer for the next tile's loads.
  auto diag_step = [&](auto bc, int s, auto fc) __attribute__((always_inline)) {
    constexpr int bi = decltype(bc)::value;
    // The first diagonal tile leaves the pipelined steps' loads in flight.
    if constexpr (decltype(fc)::value) wait_vmem_le<2 * kTileLoads>();
    else wait_vmem();
    barrier_lds();
    load_diag(s + 1, 5 - bi, s + 1 < n_dsteps);
    gemm_sdp(qbuf(bi), dobuf(bi), stbuf(bi), Int<1>{});
    mask((qt0 + s % n_diag_d) * C::kBQ);
    p_ds(stbuf(bi), pa, da);
    gemm_dvdk(qbuf(bi), dobuf(bi), pa, da);
  };
  // The first tile runs outside the loop, in straight-line code after the
  // prologue's loads, so that its partial wait is the only one.
  if (n_dsteps > 0) diag_step(Int<2>{}, 0, Int<1>{});
  for (int s = 1; s < n_dsteps; s += 2) {
    diag_step(Int<3>{}, s, Int<0>{});
    if (s + 1 < n_dsteps) diag_step(Int<2>{}, s + 1, Int<0>{});
  }
  // Buffer 3 stands for step -1 of the first pipelined step: zero it once
  // every wave is done with the diagonal tiles.
  if (n_dsteps > 0) barrier_lds();
  for (int i = threadIdx.x; i < C::kTileBytes / 16; i += 256) {
    *(__attribute__((address_space(3))) u32x4*)(qbuf(3) + 16 * i) = u32x4{0, 0, 0, 0};
    *(__attribute__((address_space(3))) u32x4*)(dobuf(3) + 16 * i) = u32x4{0, 0, 0, 0};
  }

  // ---- One pipelined step, as kNChunks chunks of kChunk products, each
  // chunk fenced from the next.  Products 0 .. NA-1 are dVᵀ/dKᵀ of step i-1
  // (ps, dt, dV then dK), products NA .. NA+NB-1 are S/dP of step i+1 (M tile
  // mt, k block ks, S then dP).  The fragment of product m is read two
  // products ahead.  P/dS of step i are cut into pieces (mt, u) of 8 queries
  // and each piece into three stages; stage g (piece g/3) runs in chunk
  // g * kChunkMt1 / (3 * kPieces), so that every piece of M tile mt is done
  // before the chunk whose products overwrite tile mt's S and dP.
  constexpr int NA = 2 * PS * DT, NB = 2 * KS * MT, NM = NA + NB;
  constexpr int kChunk = 4, kLead = 2;
  static_assert(NA % kChunk == 0 && (2 * KS) % kChunk == 0, "chunks hold whole product groups");
  constexpr int kNChunks = NM / kChunk;
  constexpr int kPieces = 2 * MT;
  constexpr int kChunkMt1 = (NA + 2 * KS * (MT - 1)) / kChunk;  // first chunk of the last M tile's S/dP
  // kNegInit (head size 128): the dP accumulators of the next step start
  // from -D, loaded in the chunk after the last stage that reads M tile mt's
  // dP (init_chunk), so that dS = P dP takes one product instead of a
  // subtraction and a product; the stages then end two chunks earlier to
  // leave the loads time before the first dP product of the last M tile.
  // Smaller heads have too few chunks and subtract D in stage 1.
  constexpr bool kNegInit = kChunkMt1 >= 4 * MT;
  constexpr int kStageEnd = kNegInit ? kChunkMt1 - 2 : kChunkMt1;
  constexpr auto stage_chunk = [](int g) constexpr { return g * kStageEnd / (3 * kPieces); };
  constexpr auto init_chunk = [](int mt) constexpr { return (3 * (2 * mt + 1) + 2) * kStageEnd / (3 * kPieces) + 1; };
  static_assert(!kNegInit || (init_chunk(0) < (NA + 1) / kChunk && init_chunk(MT - 1) < kChunkMt1),
                "-D lands in dP before its first product");

  auto fused = [&](const lds_char* stb, const lds_char* stn, const lds_char* q_old, const lds_char* do_old,
                   const lds_char* q_new, const lds_char* do_new, Frag (&pn)[PS], Frag (&dn)[PS],
                   const Frag (&po)[PS], const Frag (&dq_)[PS]) __attribute__((always_inline)) {
    float l2[kPieces][8], dd[kPieces][8], pv[kPieces][8], xv[kPieces][8];
    auto read_a = [&](auto mc) __attribute__((always_inline)) -> Frag {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NA) {
        constexpr int ps = m / (2 * DT), dt = (m % (2 * DT)) / 2, which = m % 2;
        return F::lds_col_at((which ? q_old : do_old) + 16 * ps * C::kRowBytes, coff[dt][0], coff[dt][1]);
      } else {
        constexpr int j = m - NA, mt = j / (2 * KS), ks = (j % (2 * KS)) / 2, which = j % 2;
        return F::lds_row_at((which ? do_new : q_new) + 32 * mt * C::kRowBytes, roff[ks]);
      }
    };
    auto product = [&](auto mc, const Frag& a) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NA) {
        constexpr int ps = m / (2 * DT), dt = (m % (2 * DT)) / 2, which = m % 2;
        if constexpr (which == 0) dv[dt] = E::mma(a, po[ps], dv[dt]);
        else dk[dt] = E::mma(a, dq_[ps], dk[dt]);
      } else {
        constexpr int j = m - NA, mt = j / (2 * KS), ks = (j % (2 * KS)) / 2, which = j % 2;
        if constexpr (which == 0) sv[mt] = E::mma(a, kf[ks], ks == 0 ? f32x16{} : sv[mt]);
        else dp[mt] = E::mma(a, vf[ks], (ks == 0 && !kNegInit) ? f32x16{} : dp[mt]);
      }
    };
    auto stats = [&](int pc) __attribute__((always_inline)) {
      const lds_char* sb = stb + 4 * (32 * (pc / 2) + 16 * (pc % 2));
      const u32x4 a0 = lds_read16(sb, soff), a1 = lds_read16(sb + 16, soff);
#pragma unroll
      for (int t = 0; t < 4; t++) {
        l2[pc][t] = as_float(a0[t]);
        l2[pc][4 + t] = as_float(a1[t]);
      }
      if constexpr (!kNegInit) {
        const u32x4 b0 = lds_read16(sb + 4 * C::kBQ, soff), b1 = lds_read16(sb + 4 * C::kBQ + 16, soff);
#pragma unroll
        for (int t = 0; t < 4; t++) {
          dd[pc][t] = as_float(b0[t]);  // -D
          dd[pc][4 + t] = as_float(b1[t]);
        }
      }
    };
    // Stage 0: c s - lse2; stage 1: P = exp2(.) (and dP - D without
    // kNegInit); stage 2: dS = P (dP - D), both packed, and the next piece's
    // stats read.
    auto stage = [&](auto gc) __attribute__((always_inline)) {
      constexpr int gi = decltype(gc)::value, pc = gi / 3, st = gi % 3, mt = pc / 2, u = pc % 2;
      if constexpr (st == 0) {
#pragma unroll
        for (int t = 0; t < 8; t++) xv[pc][t] = fmaf(sv[mt][8 * u + t], c, -l2[pc][t]);
      } else if constexpr (st == 1) {
#pragma unroll
        for (int t = 0; t < 8; t++) {
          pv[pc][t] = fast_exp2(xv[pc][t]);
          if constexpr (!kNegInit) xv[pc][t] = dp[mt][8 * u + t] + dd[pc][t];
        }
      } else {
#pragma unroll
        for (int t = 0; t < 8; t++) xv[pc][t] = (kNegInit ? dp[mt][8 * u + t] : xv[pc][t]) * pv[pc][t];
        pn[pc] = E::pack(pv[pc]);
        dn[pc] = E::pack(xv[pc]);
        if constexpr (pc + 1 < kPieces) stats(pc + 1);
      }
    };
    Frag ra[kLead + 1];
    stats(0);
    static_for<0, kLead>([&](auto jc) __attribute__((always_inline)) {
      ra[decltype(jc)::value] = read_a(Int<decltype(jc)::value>{});
    });
    static_for<0, kNChunks>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      static_for<0, kChunk>([&](auto jc) __attribute__((always_inline)) {
        constexpr int m = kChunk * k + decltype(jc)::value;
        if constexpr (m + kLead < NM) ra[(m + kLead) % (kLead + 1)] = read_a(Int<m + kLead>{});
        product(Int<m>{}, ra[m % (kLead + 1)]);
      });
      static_for<0, 3 * kPieces>([&](auto gc) __attribute__((always_inline)) {
        if constexpr (stage_chunk(decltype(gc)::value) == k) stage(gc);
      });
      if constexpr (kNegInit) {
        static_for<0, MT>([&](auto mc) __attribute__((always_inline)) {
          constexpr int mt = decltype(mc)::value;
          if constexpr (init_chunk(mt) == k) dp[mt] = neg_d(stn, mt);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Step i (bi = i mod 4): P/dS of step i go to (pn, dn); (po, dq_) hold
  // those of step i-1.
  auto iter = [&](auto bc, Frag (&pn)[PS], Frag (&dn)[PS], const Frag (&po)[PS], const Frag (&dq_)[PS], int i)
      __attribute__((always_inline)) {
    constexpr int bi = decltype(bc)::value;
    // Step i+1's tiles are this wave's only loads in flight; once they have
    // landed in every wave, the barrier also frees the buffer of step i-2.
    wait_vmem();
    barrier_lds();
    load_step(i + 2, (bi + 2) & 3, i + 2 < steps);
    // The lane offsets are hidden from the compiler anew every step: it then
    // adds buffer bases within the step instead of keeping a register for
    // every (buffer, offset) pair across the loop.
#pragma unroll
    for (int ks = 0; ks < KS; ks++) asm volatile("" : "+v"(roff[ks]));
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      asm volatile("" : "+v"(coff[dt][0]));
      asm volatile("" : "+v"(coff[dt][1]));
    }
    asm volatile("" : "+v"(soff));
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      asm volatile("" : "+a"(dk[dt]));
      asm volatile("" : "+a"(dv[dt]));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      asm volatile("" : "+a"(kf[ks]));
      asm volatile("" : "+a"(vf[ks]));
    }
    __builtin_amdgcn_sched_barrier(0);
    // Past the last step S/dP read a stale buffer and P/dS are never used.
    fused(stbuf(bi), stbuf((bi + 1) & 3), qbuf((bi + 3) & 3), dobuf((bi + 3) & 3), qbuf((bi + 1) & 3),
          dobuf((bi + 1) & 3), pn, dn, po, dq_);
  };

  if (n_dsteps == 0) wait_vmem_le<kTileLoads>();
  else wait_vmem();
  barrier_lds();
  if (steps > 0) gemm_sdp(qbuf(0), dobuf(0), stbuf(0), Int<kNegInit>{});
  // steps + 1 iterations: the last one only completes dV/dK of the last step.
  int i = 0;
  for (; i + 4 <= steps + 1; i += 4) {
    iter(Int<0>{}, pb, db, pa, da, i);
    iter(Int<1>{}, pa, da, pb, db, i + 1);
    iter(Int<2>{}, pb, db, pa, da, i + 2);
    iter(Int<3>{}, pa, da, pb, db, i + 3);
  }
  if (i <= steps) iter(Int<0>{}, pb, db, pa, da, i);
  if (i + 1 <= steps) iter(Int<1>{}, pa, da, pb, db, i + 1);
  if (i + 2 <= steps) iter(Int<2>{}, pb, db, pa, da, i + 2);

  const __amdgpu_buffer_rsrc_t wk = make_rsrc((char*)p.dk + kv_slab * 2, (uint32_t)Nk * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t wv = make_rsrc((char*)p.dv + kv_slab * 2, (uint32_t)Nk * C::kRowBytes);
#pragma unroll
  for (int dt = 0; dt < DT; dt++)
#pragma unroll
    for (int a4 = 0; a4 < 4; a4++) {
      const uint32_t off = (uint32_t)key * C::kRowBytes + (32 * dt + 8 * a4 + 4 * h) * 2;
      F::store4(wk, off, dk[dt][4 * a4] * p.scale, dk[dt][4 * a4 + 1] * p.scale, dk[dt][4 * a4 + 2] * p.scale,
                dk[dt][4 * a4 + 3] * p.scale);
      F::store4(wv, off, dv[dt][4 * a4], dv[dt][4 * a4 + 1], dv[dt][4 * a4 + 2], dv[dt][4 * a4 + 3]);
    }
}

// ---------------------------------------------------------------------------
// dQ (Q-outer)
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DqCfg {
  static constexpr int kWaves = 4;
  static constexpr int kBR = 32 * kWaves;
  static constexpr int kES = Elem<T>::kBytes;
  static constexpr int kRowBytes = D * kES;
  static constexpr int kBC = (kES == 4 && D == 128) ? 32 : 64;
  static constexpr int kKS = D / 16;
  static constexpr int kMT = kBC / 32;
  static constexpr int kPS = kBC / 16;
  static constexpr int kDT = D / 32;
  static constexpr int kTileBytes = kBC * kRowBytes;
};

struct DqParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse2;
  const float* dsum;
  void* dq;
  // ROWTERMS: the forward's O and LSE, from which the kernel computes its
  // rows' D_i and LSE_i*log2(e) and writes them to the workspace (lse2w,
  // dsumw: the same arrays as lse2, dsum).
  const void* o;
  const float* lse;
  float* lse2w;
  float* dsumw;
  const int* cu_q;  // packed batch: cumulative query / key counts [B + 1], else null
  const int* cu_k;
  int B, Hq, Hkv, Nq, Nk;  // Nq, Nk: the lengths (dense) or their bounds (packed)
  int tot_q, tot_k;        // packed batch: total query / key tokens
  float c;
  float scale;
};

// ROWTERMS: the kernel computes its rows' terms D_i = sum_c dO_ic O_ic and
// LSE_i * log2(e) itself (what the preprocess kernel does) and stores them in
// the workspace for a dK/dV kernel launched after it.
template <typename T, int D, bool CAUSAL, bool ROWTERMS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(DqParams p) {
  using C = DqCfg<T, D>;
  using E = Elem<T>;
  using F = Frags<T>;
  using TT = Tile<C::kRowBytes>;
  typedef typename E::Frag Frag;

  // Double-buffered K and V tiles, each buffer its own LDS object.
  __shared__ __attribute__((aligned(1024))) char k_lds0[C::kTileBytes], k_lds1[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[C::kTileBytes], v_lds1[C::kTileBytes];
  auto kbuf = [&](int par) __attribute__((always_inline)) { return (lds_char*)(par ? k_lds1 : k_lds0); };
  auto vbuf = [&](int par) __attribute__((always_inline)) { return (lds_char*)(par ? v_lds1 : v_lds0); };

  // The grid covers the longest sequence; blocks past a shorter one's last tile leave at once.
  const int bh_count = p.B * p.Hq;
  const int id = blockIdx.x;
  const int bh = id % bh_count;
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);
  const SeqRows sr = seq_rows(p.cu_q, p.cu_k, b, p.Nq, p.Nk, p.tot_q, p.tot_k);
  const int Nq = sr.nq, Nk = sr.nk;
  const int n_qt = (Nq + C::kBR - 1) / C::kBR;
  if (id / bh_count >= n_qt) return;
  const int qt = CAUSAL ? (n_qt - 1 - id / bh_count) : id / bh_count;

  const int lane = lane_id(), w = wave_id();
  const int h = lane >> 5, col = lane & 31;
  const int q0 = qt * C::kBR;
  const int qw = q0 + 32 * w;
  const int qrow = qw + col;
  const int diag = Nk - Nq;

  const size_t q_row0 = (size_t)p.Hq * sr.tq + (size_t)hq * Nq;     // first row of this (sequence, head)
  const size_t kv_row0 = (size_t)p.Hkv * sr.tk + (size_t)hkv * Nk;
  const size_t q_slab = q_row0 * D;
  const size_t kv_slab = kv_row0 * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + q_slab * C::kES, (uint32_t)Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const char*)p.dout + q_slab * C::kES, (uint32_t)Nq * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.k + kv_slab * C::kES, (uint32_t)Nk * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)p.v + kv_slab * C::kES, (uint32_t)Nk * C::kRowBytes);
  const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(p.lse2 + q_row0, (uint32_t)Nq * 4);
  const __amdgpu_buffer_rsrc_t rsd = make_rsrc(p.dsum + q_row0, (uint32_t)Nq * 4);

  int n_tiles = (Nk + C::kBC - 1) / C::kBC;
  if (CAUSAL) {
    const int last_key = min(q0 + C::kBR, Nq) - 1 + diag;
    n_tiles = last_key < 0 ? 0 : min(n_tiles, last_key / C::kBC + 1);
  }

  auto load_tile = [&](int j, int buf) __attribute__((always_inline)) {
    const uint32_t g0 = (uint32_t)j * C::kBC * C::kRowBytes;
    dma_tile<C::kRowBytes, C::kBC, C::kWaves>(rk, g0, buf ? kbuf(1) : kbuf(0), w, lane);
    dma_tile<C::kRowBytes, C::kBC, C::kWaves>(rv, g0, buf ? vbuf(1) : vbuf(0), w, lane);
  };

  if (n_tiles > 0) load_tile(0, 0);

  Frag qf[C::kKS], dof[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ks++) {
    qf[ks] = F::template global_row<D>(rq, qrow, ks, h);
    dof[ks] = F::template global_row<D>(rdo, qrow, ks, h);
  }
  float l2, dd;  // LSE_i * log2(e) and -D_i of this lane's row
  if constexpr (ROWTERMS) {
    // This lane holds elements d = 16ks + 8h + 0..7 of its row of dO; the
    // same elements of O give its half of the row sum, the lane 32 places
    // away the other half.
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((const char*)p.o + q_slab * C::kES, (uint32_t)Nq * C::kRowBytes);
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::kKS; ks++) {
      const Frag of = F::template global_row<D>(ro, qrow, ks, h);
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        // 16-bit types: one two-element dot product with float32 accumulation per pair.
        if constexpr (std::is_same_v<T, __bf16>) {
          typedef __bf16 v2 __attribute__((ext_vector_type(2)));
          part = __builtin_amdgcn_fdot2_f32_bf16(v2{dof[ks][t], dof[ks][t + 1]}, v2{of[t], of[t + 1]}, part, false);
        } else if constexpr (std::is_same_v<T, _Float16>) {
          typedef _Float16 v2 __attribute__((ext_vector_type(2)));
          part = __builtin_amdgcn_fdot2(v2{dof[ks][t], dof[ks][t + 1]}, v2{of[t], of[t + 1]}, part, false);
        } else {
          part = fmaf(dof[ks].v[t], of.v[t], part);
          part = fmaf(dof[ks].v[t + 1], of.v[t + 1], part);
        }
      }
    }
    dd = -sum_halves(part);  // the workspace holds -D
    const float L = as_float(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.lse + q_row0, (uint32_t)Nq * 4),
                                                                  (uint32_t)qrow * 4, 0, 0));
    // Rows that see no key carry LSE = -inf; +inf makes exp2(s - lse2) vanish.
    l2 = L == -INFINITY ? INFINITY : L * kLog2e;
    if (h == 0) {
      buf_store4(make_rsrc(p.dsumw + q_row0, (uint32_t)Nq * 4), (uint32_t)qrow * 4, __builtin_bit_cast(uint32_t, dd));
      buf_store4(make_rsrc(p.lse2w + q_row0, (uint32_t)Nq * 4), (uint32_t)qrow * 4, __builtin_bit_cast(uint32_t, l2));
    }
  } else {
    l2 = as_float(__builtin_amdgcn_raw_buffer_load_b32(rs2, (uint32_t)qrow * 4, 0, 0));
    dd = as_float(__builtin_amdgcn_raw_buffer_load_b32(rsd, (uint32_t)qrow * 4, 0, 0));
  }

  f32x16 dq[C::kDT];
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++) dq[dt] = f32x16{};

  // Per-lane LDS offsets of the K / V row fragments (A rows are sigma-permuted
  // keys) and of the Kᵀ column fragments.
  uint32_t roff[C::kKS], coff[C::kDT][2];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ks++) roff[ks] = F::template row_off<TT>(sigma(col), ks, h);
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++)
#pragma unroll
    for (int u = 0; u < 2; u++) coff[dt][u] = F::template col_off<TT>(32 * dt, u, lane);

  wait_vmem();
  barrier_lds();

  auto tile = [&](int j, const lds_char* kb, const lds_char* vb) __attribute__((always_inline)) {
    const int k0 = j * C::kBC;
    if (CAUSAL && k0 > qw + 31 + diag) return;
    // ---- Sᵀ = K Qᵀ and dPᵀ = V dOᵀ; A rows are sigma-permuted keys.
    f32x16 sv[C::kMT], dp[C::kMT];
    // dPᵀ starts from -D (the same for every register of a lane: its query
    // row), so the products leave dPᵀ - D.
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++) {
      sv[mt] = f32x16{};
#pragma unroll
      for (int r = 0; r < 16; r++) dp[mt][r] = dd;
    }
#pragma unroll
    for (int ks = 0; ks < C::kKS; ks++) {
#pragma unroll
      for (int mt = 0; mt < C::kMT; mt++) {
        if constexpr (C::kES == 2) {
          sv[mt] = E::mma(F::lds_row_at(kb + 32 * mt * C::kRowBytes, roff[ks]), qf[ks], sv[mt]);
          dp[mt] = E::mma(F::lds_row_at(vb + 32 * mt * C::kRowBytes, roff[ks]), dof[ks], dp[mt]);
        } else {
          const int row = 32 * mt + sigma(col);
          sv[mt] = E::mma(F::template lds_row<TT>(kb, row, ks, h), qf[ks], sv[mt]);
          dp[mt] = E::mma(F::template lds_row<TT>(vb, row, ks, h), dof[ks], dp[mt]);
        }
      }
    }
    if constexpr (C::kES == 2) sched_reads_ahead<2 * C::kKS * C::kMT, 2 * C::kKS * C::kMT, 4>();
    // ---- dSᵀ = Pᵀ ∘ (dPᵀ - D).  Register r of tile mt holds key
    //      k0 + 32*mt + 16*(r/8) + 8h + (r%8).  Keys past Nk are masked too
    //      (their zero-filled rows must not meet an infinite P).
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) sv[mt][r] = fast_exp2(fmaf(sv[mt][r], p.c, -l2));
    // Only tiles cut by Nk or by the causal diagonal mask P (a uniform branch).
    if ((k0 + C::kBC > Nk) || (CAUSAL && k0 + C::kBC - 1 > qw + diag)) {
      const int horizon = CAUSAL ? min(qrow + diag, Nk - 1) : Nk - 1;
#pragma unroll
      for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
        for (int r = 0; r < 16; r++)
          if (k0 + 32 * mt + 16 * (r >> 3) + 8 * h + (r & 7) > horizon) sv[mt][r] = 0.f;
    }
#pragma unroll
    for (int mt = 0; mt < C::kMT; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) dp[mt][r] = sv[mt][r] * dp[mt][r];
    // ---- dQᵀ += Kᵀ dSᵀ (column = query, k = key).
#pragma unroll
    for (int ps = 0; ps < C::kPS; ps++) {
      float dsv[8];
#pragma unroll
      for (int t = 0; t < 8; t++) dsv[t] = dp[ps >> 1][8 * (ps & 1) + t];
      const Frag dsf = E::pack(dsv);
#pragma unroll
      for (int dt = 0; dt < C::kDT; dt++) {
        if constexpr (C::kES == 2)
          dq[dt] = E::mma(F::lds_col_at(kb + 16 * ps * C::kRowBytes, coff[dt][0], coff[dt][1]), dsf, dq[dt]);
        else
          dq[dt] = E::mma(F::template lds_col<TT>(kb, 16 * ps, 32 * dt, lane), dsf, dq[dt]);
      }
    }
    if constexpr (C::kES == 2) sched_reads_ahead<2 * C::kPS * C::kDT, C::kPS * C::kDT, 4>();
  };

  if constexpr (C::kES == 2) {
    // Two tiles per trip so that every buffer is a compile-time LDS object.
    for (int j = 0; j < n_tiles; j += 2) {
      if (j + 1 < n_tiles) load_tile(j + 1, 1);
      tile(j, kbuf(0), vbuf(0));
      wait_vmem();
      barrier_lds();
      if (j + 1 < n_tiles) {
        if (j + 2 < n_tiles) load_tile(j + 2, 0);
        tile(j + 1, kbuf(1), vbuf(1));
        wait_vmem();
        barrier_lds();
      }
    }
  } else {
    for (int j = 0; j < n_tiles; j++) {
      const int buf = j & 1;
      if (j + 1 < n_tiles) load_tile(j + 1, buf ^ 1);
      tile(j, kbuf(buf), vbuf(buf));
      wait_vmem();
      barrier_lds();
    }
  }

  const __amdgpu_buffer_rsrc_t wq = make_rsrc((char*)p.dq + q_slab * C::kES, (uint32_t)Nq * C::kRowBytes);
#pragma unroll
  for (int dt = 0; dt < C::kDT; dt++)
#pragma unroll
    for (int a4 = 0; a4 < 4; a4++) {
      const int d0 = 32 * dt + 8 * a4 + 4 * h;
      F::store4(wq, (uint32_t)qrow * C::kRowBytes + d0 * C::kES, dq[dt][4 * a4] * p.scale,
                dq[dt][4 * a4 + 1] * p.scale, dq[dt][4 * a4 + 2] * p.scale, dq[dt][4 * a4 + 3] * p.scale);
    }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
// Phase launchers.  The workspace holds D (rows floats) then lse2 (rows floats).
// Query rows of the batch (of every head): dense B*Hq*Nq, packed Hq*tot_q.
int64_t query_rows(const BwdArgs& a) { return a.cu_q ? (int64_t)a.Hq * a.tot_q : (int64_t)a.B * a.Hq * a.Nq; }

template <typename T, int D>
hipError_t launch_prep(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = query_rows(a);
  if (rows == 0) return hipSuccess;
  constexpr int kTPR = D / (16 / (int)sizeof(T));
  const int64_t threads = rows * kTPR;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3(grid), dim3(256), 0, stream, (const T*)a.o, (const T*)a.dout,
                     a.lse, a.dsum, a.dsum + rows, rows);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_dkdv(const BwdArgs& a, hipStream_t stream) {
  using C = DkvCfg<T, D>;
  const int64_t rows = query_rows(a);
  DkvParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout; p.lse2 = a.dsum + rows; p.dsum = a.dsum;
  p.dk = a.dk; p.dv = a.dv;
  p.cu_q = a.cu_q; p.cu_k = a.cu_k;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.tot_q = a.tot_q; p.tot_k = a.tot_k;
  p.c = a.scale * kLog2e; p.scale = a.scale;
  const ExpScale es = exp_scale(p.c);
  p.c_mag = es.c; p.neg_k = es.neg_q;
  const unsigned grid = (unsigned)((a.Nk + C::kBKV - 1) / C::kBKV) * a.B * a.Hkv;
  if (grid == 0) return hipSuccess;  // a packed batch with no key
  // 16-bit types take the pipelined kernel; float32 (whose fragments leave
  // no registers for a pipeline) the plain one.
  if constexpr (Elem<T>::kBytes == 2)
    hipLaunchKernelGGL((bwd_dkdv16_kernel<T, D, CAUSAL>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, bool ROWTERMS>
hipError_t launch_dq(const BwdArgs& a, hipStream_t stream) {
  using C = DqCfg<T, D>;
  const int64_t rows = query_rows(a);
  DqParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout; p.lse2 = a.dsum + rows; p.dsum = a.dsum; p.dq = a.dq;
  p.o = a.o; p.lse = a.lse; p.lse2w = a.dsum + rows; p.dsumw = a.dsum;
  p.cu_q = a.cu_q; p.cu_k = a.cu_k;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.tot_q = a.tot_q; p.tot_k = a.tot_k;
  p.c = a.scale * kLog2e; p.scale = a.scale;
  const unsigned grid = (unsigned)((a.Nq + C::kBR - 1) / C::kBR) * a.B * a.Hq;
  if (grid == 0) return hipSuccess;  // a packed batch with no query
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, ROWTERMS>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_phases(const BwdArgs& a, int phases, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (phases & kBwdDqRowTerms) {
    // dQ with the row terms first, then dK/dV, which reads them.
    if ((e = launch_dq<T, D, CAUSAL, true>(a, stream)) != hipSuccess) return e;
    if ((phases & kBwdDkdv) && (e = launch_dkdv<T, D, CAUSAL>(a, stream)) != hipSuccess) return e;
    return e;
  }
  if ((phases & kBwdPrep) && (e = launch_prep<T, D>(a, stream)) != hipSuccess) return e;
  if ((phases & kBwdDkdv) && (e = launch_dkdv<T, D, CAUSAL>(a, stream)) != hipSuccess) return e;
  if ((phases & kBwdDq) && (e = launch_dq<T, D, CAUSAL, false>(a, stream)) != hipSuccess) return e;
  return e;
}

template <typename T>
hipError_t launch_dtype(const BwdArgs& a, int phases, hipStream_t s) {
  switch (a.d) {
    case 32: return a.causal ? launch_phases<T, 32, true>(a, phases, s) : launch_phases<T, 32, false>(a, phases, s);
    case 64: return a.causal ? launch_phases<T, 64, true>(a, phases, s) : launch_phases<T, 64, false>(a, phases, s);
    case 128: return a.causal ? launch_phases<T, 128, true>(a, phases, s) : launch_phases<T, 128, false>(a, phases, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int phases, hipStream_t stream) {
  switch (a.dtype) {
    case 0: return launch_dtype<float>(a, phases, stream);
    case 1: return launch_dtype<_Float16>(a, phases, stream);
    case 2: return launch_dtype<__bf16>(a, phases, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
