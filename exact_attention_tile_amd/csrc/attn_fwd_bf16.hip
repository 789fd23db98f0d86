// bf16 tiled exact attention forward for gfx950 (MI355X, CDNA4).
//
// What it computes: O = softmax(Q K^T * scale) V and lse = ln sum exp(scores)
// per query row, on [B][N][H][d] tensors ("FlashAttention-4 no Blackwell
// B200 ...", section "Por que o Blackwell exige mais do que multiplicações
// rápidas"), tile by tile with an online softmax so the N x N scores stay on
// chip (dev.to "FlashAttention-4 em Blackwell B200", sections 1 and 4), with
// the threshold-gated rescale of "FlashAttention 4: Atenção Mais Rápida ...",
// section "Reescalonamento Softmax Online Mais Inteligente".
//
// Work decomposition
//   one work-group = NW waves = 32*NW query rows of one (batch, head);
//   one wave       = 32 query rows, for which it owns the output tile;
//   K/V tiles of BC keys are streamed HBM -> LDS (global_load_lds, no
//   registers), double buffered, two barriers per tile (see below).
//
// Transposed formulation.  Each wave computes S^T = K_j Q^T with
// v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T kept in VGPRs for
// the whole kernel).  In the 32x32 accumulator layout lane l holds column
// l%32 -- one query -- and 16 of the 32 key rows (row 8*(r/4)+4*(l/32)+r%4 for
// register r).  So the row max and row sum of the softmax are in-lane
// reductions plus one exchange with lane l^32 (permlane32_swap), the rescale
// factor is a per-lane scalar on that lane's output registers, and the
// exponentials, converted to bf16, are already in the B-operand layout of the
// second product O^T += V_j^T P^T: B slot t of lane-half h holds key
// pi(h,t) = 4h + (t&3) + 8*(t>>2) of a 16-key group.  The matching A operand
// (V^T, 8 keys x 1 column per lane) comes straight from the row-major V tile
// with two ds_read_b64_tr_b16 (transposing LDS reads of 4 rows x 16 columns
// per 16-lane group).
//
// Overlap between the two waves of a SIMD (ping-pong).  Waves i and i+4 of
// the work-group share a SIMD; waves 0-3 form group A and waves 4-7 group B.
// The tile loop runs in phases separated by work-group barriers, two per
// K/V tile, and group B runs one phase behind group A.  Each wave alternates
//   X_j : S^T of tile j+1 = K_{j+1} Q^T and O^T += V_j^T P_j^T  (matrix cores)
//   Y_j : row max, gated rescale and exponentials of tile j+1   (vector ALU)
// so in every phase one wave of each SIMD is on the matrix cores while the
// other is on the vector ALU; the matrix-core wave raises its issue priority
// (s_setprio) for the phase, so the MFMAs are never queued behind the
// partner's vector work.  Group B also issues the LDS-bound loads in its
// Y phases, two phases before the data is needed.
//
// Softmax in base 2: scores are kept as s*c with c = |scale|*log2(e) folded
// into one fma; p = exp2(s*c - m_ref) on v_exp_f32.  m_ref only moves when a
// tile's row maximum exceeds it by more than TAU (log2 units), so p <= 2^TAU
// and most tiles skip the O rescale; the skip is decided per wave (ballot).
// The row sum adds the fp32 p (rounding p to bf16 first would cost the
// log-sum-exp up to 2^-9 relative in l).
#include <type_traits>

#include "attn_kernels.hpp"

namespace attn {

constexpr float kTauBf16 = 8.0f;  // p <= 256: exact range for bf16 / fp32
constexpr float kPMaxBf16 = 256.0f;   // 2^kTauBf16

// 16-byte-chunk XOR swizzles of the row-major [BC][D] LDS tiles.
//  K: a ds_read_b128 A-operand read has 16 lanes on 16 consecutive rows at
//     one chunk -> the swizzle spreads them over all 64 banks.
//  V: a ds_read_b64_tr_b16 read has each 32 lanes on 4 consecutive rows x 4
//     consecutive chunks -> the swizzle moves each row's 64 bytes to a
//     distinct quarter of the bank space.
template <int D> __device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D> __device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

template <int D, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwd_bf16_kernel(FwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(BC == 64 || BC == 128, "kv tile");
  static_assert(NW == 8, "two groups of four waves, one wave of each per SIMD");
  constexpr int BR = NW * 32;            // query rows per work-group
  constexpr int NKB = BC / 32;           // 32-key blocks per tile
  constexpr int NDB = D / 32;            // 32-wide column blocks of the output
  constexpr int NKS = D / 16;            // k-steps of the QK^T product
  constexpr int NKK = BC / 16;           // 16-key steps of the P.V product
  constexpr int TILE = BC * D;           // elements per K or V tile

  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * TILE];
  __bf16* ks_base = smem;                // K tiles: [2][BC][D]
  __bf16* vs_base = smem + 2 * TILE;     // V tiles: [2][BC][D]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;             // 0: group A, 1: group B
  const int ln = lane & 31;
  const int lh = lane >> 5;

  // one work item (batch*head, query tile) per step; the loop runs once
  // unless the launch is persistent.  The item's first loads go into LDS
  // only after every wave has passed the previous item's last barrier.
  for (int step = 0;; ++step) {
  int L;
  if (!item_of(p, step, L)) break;
  int bh, qt;
  block_to_work(p, L, bh, qt);
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  SeqView sv;
  if (!seq_view(p, D, b, h, qt * BR, sv)) continue;   // whole work-group, before any barrier
  const int N = sv.N;
  const long long tok = (long long)p.H * D;       // elements between tokens of Q and O
  const long long tkv = (long long)p.Hkv * D;     // elements between tokens of K and V

  const int q0 = qt * BR;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + ln;

  const __bf16* __restrict__ qg = (const __bf16*)p.q + sv.q_base;
  const __bf16* __restrict__ kg = (const __bf16*)p.k + sv.kv_base;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + sv.kv_base;

  // ---- Q^T fragments (B operand): lane (n=ln, h=lh) holds Q[myq][16ks+8lh .. +7]
  bf16x8 qf[NKS];
  {
    const int qr = myq < N ? myq : N - 1;
    const u32x4* src = (const u32x4*)(qg + (long long)qr * tok + 8 * lh);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 t = src[2 * ks];
      t ^= p.qsign;
      qf[ks] = __builtin_bit_cast(bf16x8, t);
    }
  }

  // ---- tile range of this work-group and of this wave
  const int n_kv_all = (N + BC - 1) / BC;
  int wg_tiles = n_kv_all;
  int wv_tiles = qw0 < N ? n_kv_all : 0;
  if (CAUSAL) {
    const int last_wg = min(q0 + BR - 1, N - 1);
    wg_tiles = last_wg / BC + 1;
    if (qw0 < N) wv_tiles = min(qw0 + 31, N - 1) / BC + 1;
  }

  // ---- tile loader (group B only): global_load_lds_dwordx4 straight into
  // the swizzled LDS tile (lds_dma_*).  One instruction fills 1 KiB of LDS,
  // lane l writing bytes [16 l, 16 l + 16) after the wave-uniform base, so
  // the swizzle is applied by choosing each lane's source chunk.  Rows past
  // N are clamped to row N-1: their keys are masked, so they contribute
  // p = 0 against finite V.  Completion is awaited explicitly (vmcnt) before
  // a barrier.  A wave's four loads of a tile share one M0 value, so each
  // lane's offset for load i is stored less 1024 i (still >= 0: load i
  // starts 1024 i bytes into the LDS tile, and at least that many bytes of
  // global rows into the tile).
  constexpr int LPW = TILE * 2 / 1024 / 4;              // loads per B wave per tensor per tile
  static_assert(LPW == 4 && LPW * 1024 * 4 == TILE * 2, "tile must split into four 1 KiB loads per wave");
  const int wb = wave & 3;                               // index within the group
  int ld_row[LPW];
  unsigned kgo[LPW], vgo[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int off = (wb * LPW + i) * 512 + lane * 8;     // element offset in the tile
    const int row = off / D;
    const int pc = (off - row * D) / 8;                   // physical 16-byte chunk
    ld_row[i] = row;
    kgo[i] = (unsigned)(((long long)row * tkv + (pc ^ swz_k<D>(row)) * 8) * 2) - (unsigned)(i * 1024);
    vgo[i] = (unsigned)(((long long)row * tkv + (pc ^ swz_v<D>(row)) * 8) * 2) - (unsigned)(i * 1024);
  }
  const unsigned lds_k = (unsigned)(size_t)((ATTN_LDS __bf16*)ks_base);
  const unsigned lds_v = (unsigned)(size_t)((ATTN_LDS __bf16*)vs_base);
  const unsigned lds_wave = __builtin_amdgcn_readfirstlane((unsigned)(wb * LPW * 1024));
  // The loads' addresses are scalar work of the loading wave's vector phase,
  // where a lone wave issues every instruction slowly: a tile's byte offset
  // is one 32x32 -> 64-bit product of the tile index and the tile's bytes
  // (BC tokens of K or V), and a full tile is one compare against the
  // count of full tiles.
  const unsigned tile_bytes = (unsigned)(BC * 2) * (unsigned)tkv;
  const int n_full = N / BC;
  // a full tile: the wave's four loads from the tile at global address base
  auto load_full = [&](const unsigned* go, const void* base, unsigned la0) {
    lds_dma_s<LPW>(la0, go, base);
  };
  auto load_tile = [&](const unsigned* go, const __bf16* src, unsigned lds_buf, int j) {
    const int kv0 = j * BC;
    const unsigned la0 = lds_buf + lds_wave;
    if (__builtin_expect(j < n_full, 1)) {
      load_full(go, (const char*)src + (unsigned long long)(unsigned)j * tile_bytes, la0);
    } else {
      // ragged last tile: clamp the rows (64-bit addresses)
      const __bf16* base = src + (long long)kv0 * tkv;
      const void* g[LPW];
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const long long back = (long long)(kv0 + ld_row[i] < N ? 0 : kv0 + ld_row[i] - (N - 1)) * tkv;
        g[i] = base + (long long)(go[i] / 2) - back;
      }
      lds_dma_v<LPW>(la0, g);
    }
  };
  auto load_k = [&](int j) { load_tile(kgo, kg, lds_k + (unsigned)((j & 1) * TILE * 2), j); };
  auto load_v = [&](int j) { load_tile(vgo, vg, lds_v + (unsigned)((j & 1) * TILE * 2), j); };
  auto wait_loads = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // ---- per-lane LDS read offsets (elements)
  // K A-operand: row kb*32+ln, chunk 2ks+lh (swizzled by the row)
  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = ln * D + (((2 * ks + lh) ^ swz_k<D>(ln)) * 8);
  // V^T A-operand via the transposing read: in each 16-lane group, source
  // lane i reads row key0 + i/4, columns d0 + 4*(i%4) .. +3.
  const int gi = lane & 15;
  const int vrow_l = 4 * lh + (gi >> 2);                  // row within a 16-key group (half 0)
  const int vsw = swz_v<D>(vrow_l);                        // rows differ by multiples of 4 -> constant
  int voff[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int chunk = 4 * db + ((lane & 16) >> 3) + ((gi & 3) >> 1);
    voff[db] = vrow_l * D + ((chunk ^ vsw) * 8) + (gi & 1) * 4;
  }

  // ---- running state
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_ref = -__builtin_inff();   // reference max, log2 units
  float l_part[2] = {0.f, 0.f};      // this lane-half's share of the row sum (2 chains)
  const float c = p.c;
  f32x16 s[NKB];                     // S^T of the tile whose softmax is next
  bf16x8 pf[NKK];                    // P of the tile whose P.V is next
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) pf[kk] = bf16x8{};

  // ---- X_j: S^T of tile j+1 (K tile kt) and O^T += V_j^T P_j^T (V tile vt)
  auto phase_x = [&](auto qk_tag, auto pv_tag, const __bf16* kt, const __bf16* vt)
                     __attribute__((always_inline)) {
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr bool PV = decltype(pv_tag)::value;
    // the matrix-core phase issues first on its SIMD; the partner wave's
    // vector ALU work fills the remaining issue slots.  One stream of
    // products, the S^T ones (ks-major) then the P.V ones, each operand read
    // from LDS PF products ahead of its MFMA (a fence after every MFMA keeps
    // that order whatever code surrounds the phase).
    constexpr int PF = 6;
    constexpr int NQ = QK ? NKS * NKB : 0;
    constexpr int NP = NQ + (PV ? NKK * NDB : 0);
    bf16x8 a[NP];
    auto rd = [&](int i) __attribute__((always_inline)) {
      if (i < NQ) {
        const int ks = i / NKB, kb = i % NKB;
        a[i] = *(const bf16x8*)(kt + kb * 32 * D + koff[ks]);
      } else {
        const int kk = (i - NQ) / NDB, db = (i - NQ) % NDB;
        const __bf16* vb = vt + kk * 16 * D + voff[db];
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(vb));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(vb + 8 * D));
        i32x4 w;
        w[0] = (int)(unsigned short)lo[0] | ((int)(unsigned short)lo[1] << 16);
        w[1] = (int)(unsigned short)lo[2] | ((int)(unsigned short)lo[3] << 16);
        w[2] = (int)(unsigned short)hi[0] | ((int)(unsigned short)hi[1] << 16);
        w[3] = (int)(unsigned short)hi[2] | ((int)(unsigned short)hi[3] << 16);
        a[i] = __builtin_bit_cast(bf16x8, w);
      }
    };
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int i = 0; i < PF && i < NP; ++i) rd(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + PF < NP) rd(i + PF);
      if (i < NQ) {
        const int ks = i / NKB, kb = i % NKB;
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qf[ks], ks == 0 ? f32x16{} : s[kb], 0,
                                                       0, 0);
      } else {
        const int kk = (i - NQ) / NDB, db = (i - NQ) % NDB;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], pf[kk], oacc[db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- Y_j: softmax of S_{j+1} (keys kv0 ..): mask, gated rescale of
  // m_ref / l / O, exponentials -> pf.
  //
  // p = exp2(s c - m_ref) of the tile, rounded to bf16 into pf, and two
  // partial row sums t of the fp32 p (this lane-half's keys).  s is kept.
  // hook(i) runs after the i-th group of eight packed values (the loading
  // group issues its tile loads there).
  auto exponentials = [&](float* t, auto&& hook) __attribute__((always_inline)) {
    const float neg_m = -m_ref;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = half * 8 + 2 * i;
          const float e0 = fast_exp2(__builtin_fmaf(s[kb][r], c, neg_m));
          const float e1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], c, neg_m));
          w[i] = pack_bf16x2(e0, e1);
          if (kb == 0 && half == 0 && i == 0) {
            t[0] = e0;
            t[1] = e1;
          } else {
            t[0] += e0;
            t[1] += e1;
          }
        }
        pf[kb * 2 + half] = __builtin_bit_cast(bf16x8, w);
        // the packs are used here, so the compiler does not sink them below
        // the rescale branch that follows (which would keep every p live
        // across it)
        asm volatile("" ::"v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]));
        hook(kb * 2 + half);
      }
    }
  };
  // Row maximum and gated rescale: m = max_j s_j c over the tile; where it
  // exceeds m_ref by more than TAU, m_ref moves to it and l and O are scaled
  // by exp2(m_ref_old - m).  Afterwards every p of the tile is at most 2^TAU.
  auto rescale = [&]() __attribute__((always_inline)) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[kb][r]), s[kb][r + 1]);
    mx = pair_max(mx);
    const float mt = mx * c;
    const bool need = mt > m_ref + kTauBf16;
    const float alpha = need ? fast_exp2(m_ref - mt) : 1.f;
    m_ref = need ? mt : m_ref;
    l_part[0] *= alpha;
    l_part[1] *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    __builtin_amdgcn_sched_barrier(0);
  };
  auto no_hook = [](int) {};
  auto phase_y = [&](auto masked_tag, int kv0, auto first_tag, auto&& hook) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;   // the wave's first tile: m_ref = -inf
    if constexpr (MASKED) {
      // key kv0 + off (off = kb*32 + 8*(r/4) + 4*lh + r%4) is visible iff
      // off - 4*lh <= lim
      const int lim = min(CAUSAL ? myq - kv0 - 4 * lh : 0x7fffffff, N - 1 - kv0 - 4 * lh);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -__builtin_inff();
    }
    // The gate without the row maximum on the common path: the tile's
    // exponentials are taken against the current m_ref first.  When every
    // lane's partial sum of its p is at most 2^TAU, so is every p -- and a
    // maximum more than TAU above m_ref would give a p above 2^TAU -- so no
    // row needs the rescale and the tile is kept.  Otherwise (inf or NaN
    // sums included) the wave takes the row maximum, applies the gate and
    // redoes the tile.  A wave's first tile, with no reference yet, takes
    // the maximum right away.
    float t[2];
    if constexpr (FIRST) {
      // no reference yet: the sums would be inf or NaN, so take the maximum
      // right away
      rescale();
      exponentials(t, hook);
    } else {
      exponentials(t, hook);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(t[0] + t[1] <= kPMaxBf16)) != 0, 0)) {
        rescale();
        exponentials(t, no_hook);
      }
    }
    l_part[0] += t[0];
    l_part[1] += t[1];
  };

  // ---- phase schedule ------------------------------------------------------
  // Group A runs X_j in phase 2j+2 and Y_j in phase 2j+3; group B one phase
  // later.  So K_t is read in phases 2t and 2t+1 and V_t in phases 2t+2 and
  // 2t+3 (from buffer t&1).  Group B loads K_{u+1} and V_u in its vector
  // phase 2u (into buffers last read in phases 2u-2 / 2u-1) and
  // waits for them at the end of phase 2u+1.  Every wave passes the same
  // number of phase barriers, 2 * wg_tiles + 2.
  //
  // A wave with T = wv_tiles tiles runs X_{-1} (S of tile 0 only), Y_{-1},
  // then X_j (both products) and Y_j for j = 0 .. T-2, then X_{T-1} (P.V
  // only), and idles to the last phase.  Only the wave's last tile can need
  // the mask (the causal diagonal, a ragged end), so the tiles before the
  // first masked one run in a loop without it.  The two groups run separate
  // copies of the schedule, so group B's loads and waits sit at fixed points
  // of its phases.
  using T_ = std::true_type;
  using F_ = std::false_type;
  const int n_phases = 2 * wg_tiles + 2;
  auto loads_for = [&](int u) {
    u = __builtin_amdgcn_readfirstlane(u);    // an SGPR for the loads' addresses
    if (__builtin_expect(u + 1 < wg_tiles, 1)) load_k(u + 1);
    if (__builtin_expect(u < wg_tiles, 1)) load_v(u);
  };
  auto kt_of = [&](int j) { return ks_base + ((j + 1) & 1) * TILE; };   // K tile of X_j
  auto vt_of = [&](int j) { return vs_base + (j & 1) * TILE; };         // V tile of X_j

  if (grp == 1 && wg_tiles > 0) load_k(0);
  wait_loads();
  __syncthreads();

  const int T = wv_tiles;
  // first tile that needs the mask: the causal diagonal or the ragged end
  int first_masked = N / BC;
  if (CAUSAL) first_masked = min(first_masked, (qw0 + 1) / BC);
  const int t_plain = min(first_masked, T);
  auto schedule = [&](auto loader_tag) __attribute__((always_inline)) {
    constexpr bool LOADER = decltype(loader_tag)::value;   // group B
    int ph = 0;
    // Y phases start with group B's loads, X phases end with its wait
    auto y_start = [&]() {
      if constexpr (LOADER) loads_for(ph >> 1);
    };
    auto x_end = [&]() {
      if constexpr (LOADER) wait_loads();
      __syncthreads();
      ++ph;
    };
    auto y_end = [&]() {
      __syncthreads();
      ++ph;
    };
    if constexpr (LOADER) {                       // group B starts one phase later
      y_start();
      y_end();
    }
    if (T > 0) {
      phase_x(T_{}, F_{}, kt_of(-1), vt_of(-1));
      x_end();
      y_start();
      if (first_masked <= 0)
        phase_y(T_{}, 0, T_{}, no_hook);
      else
        phase_y(F_{}, 0, T_{}, no_hook);
      y_end();
      // X_{t-1}, Y_{t-1} (softmax of tile t), unmasked.  At d = 128 the loop
      // is unrolled by two so that each step's buffers are compile-time
      // constants, folded into the LDS reads' offsets (t is odd in the first
      // step); that takes the address arithmetic out of the matrix-core
      // phase.  At d = 64 the unrolled form measured slower.
      auto plain_step = [&](auto odd_tag, int t) __attribute__((always_inline)) {
        constexpr bool ODD = decltype(odd_tag)::value;
        phase_x(T_{}, T_{}, ks_base + (ODD ? TILE : 0), vs_base + (ODD ? 0 : TILE));
        x_end();
        y_start();
        phase_y(F_{}, t * BC, F_{}, no_hook);
        y_end();
      };
      int t = 1;
      // d = 128: steps whose two loads (K_{t+2}, V_{t+1}) are full tiles
      // inside the work-group's range take them without tests, the global
      // bases as running pointers: the loading wave issues its vector phase
      // alone, so each scalar instruction and branch there costs it issue
      // time.  Each tensor's four loads go out after a group of packed values
      // (K after the first, V after the second) rather than all at the phase
      // start: 1.5-3% faster on every d = 128 workload.
      const int t_fast = LOADER ? min(t_plain, min(n_full, wg_tiles) - 2) : 0;
      const char* kp = (const char*)kg + (unsigned long long)(unsigned)(t + 2) * tile_bytes;
      const char* vp = (const char*)vg + (unsigned long long)(unsigned)(t + 1) * tile_bytes;
      // K_{t+2} goes to buffer t & 1, V_{t+1} to buffer (t + 1) & 1
      auto fast_step = [&](int t, const __bf16* kt, const __bf16* vt, unsigned lk, unsigned lv)
                           __attribute__((always_inline)) {
        phase_x(T_{}, T_{}, kt, vt);
        x_end();
        // with no branch here, the scheduler would hoist the softmax above
        // the barrier into the matrix-core phase
        __builtin_amdgcn_sched_barrier(0);
        auto hook = [&](int i) __attribute__((always_inline)) {
          if (i == 0) load_full(kgo, kp, lk);
          if (i == 1) load_full(vgo, vp, lv);
        };
        phase_y(F_{}, t * BC, F_{}, hook);
        kp += tile_bytes;
        vp += tile_bytes;
        y_end();
      };
      if constexpr (D == 128) {
        if constexpr (LOADER) {
          for (; t + 1 < t_fast; t += 2) {
            fast_step(t, ks_base + TILE, vs_base, lds_k + lds_wave + TILE * 2,
                      lds_v + lds_wave);
            fast_step(t + 1, ks_base, vs_base + TILE, lds_k + lds_wave,
                      lds_v + lds_wave + TILE * 2);
          }
        }
        for (; t + 1 < t_plain; t += 2) {
          plain_step(T_{}, t);
          plain_step(F_{}, t + 1);
        }
        if (t < t_plain) {
          plain_step(T_{}, t);
          ++t;
        }
      } else {
        // (the same fast steps at d = 64, with run-time buffers, measured
        // 5% slower)
        for (; t < t_plain; ++t) {
          phase_x(T_{}, T_{}, kt_of(t - 1), vt_of(t - 1));
          x_end();
          y_start();
          phase_y(F_{}, t * BC, F_{}, no_hook);
          y_end();
        }
      }
      for (; t < T; ++t) {              // the masked tail
        phase_x(T_{}, T_{}, kt_of(t - 1), vt_of(t - 1));
        x_end();
        y_start();
        phase_y(T_{}, t * BC, F_{}, no_hook);
        y_end();
      }
      phase_x(F_{}, T_{}, kt_of(T - 1), vt_of(T - 1));
      x_end();
    }
    // idle to the last phase (group B keeps loading for the other waves)
    for (; ph < n_phases;) {
      if (LOADER && (ph & 1) == 0) {
        y_start();
        y_end();
      } else {
        x_end();
      }
    }
  };
  if (grp == 1)
    schedule(T_{});
  else
    schedule(F_{});

  // ---- epilogue: O = acc / l -> bf16, lse = ln2 * (m_ref + log2 l)
  const float l_tot = pair_sum(l_part[0] + l_part[1]);   // wave-uniform, before any lane test
  if (myq < N) {
    const float inv = 1.f / l_tot;
    __bf16* og = (__bf16*)p.o + sv.q_base + (long long)myq * tok;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * lh;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *(u32x2*)(og + d0) = w;
      }
    }
    if (lh == 0) {
      p.lse[sv.lse_base + myq] = (m_ref + fast_log2(l_tot)) * 0.69314718055994531f;
    }
  }
  }   // work items
}

// ---------------------------------------------------------------------------
// host-side launch helpers (called by the C ABI in attn_api.cpp)
// ---------------------------------------------------------------------------
template <int D, int NW, int BC, bool CAUSAL>
static hipError_t launch_bf16_t(const FwdParams& prm, int grid, hipStream_t stream) {
  return launch_kernel(attn_fwd_bf16_kernel<D, NW, BC, CAUSAL>, dim3(grid), dim3(NW * 64), stream,
                       prm);
}

// Waves per work-group: 8 (two per SIMD, one of each ping-pong group).
// Keys per K/V tile: 64 at d = 128 (the S/P registers of a 128-key tile do
// not fit next to the d = 128 accumulators); 128 at d = 64, which halves the
// barriers per key.
constexpr int kBf16Waves = 8;

int bf16_rows_per_block(int d) { return kBf16Waves * 32; }

hipError_t launch_bf16(const FwdParams& prm, int d, int causal, int grid, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch_bf16_t<128, kBf16Waves, 64, true>(prm, grid, stream)
                  : launch_bf16_t<128, kBf16Waves, 64, false>(prm, grid, stream);
  }
  return causal ? launch_bf16_t<64, kBf16Waves, 128, true>(prm, grid, stream)
                : launch_bf16_t<64, kBf16Waves, 128, false>(prm, grid, stream);
}

}  // namespace attn
