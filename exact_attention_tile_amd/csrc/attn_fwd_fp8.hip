// OCP FP8 E4M3 tiled exact attention forward for gfx950 (MI355X, CDNA4).
//
// Same method, work decomposition and wave schedule as the bf16 kernel
// (attn_fwd_bf16.hip): online softmax over K/V tiles with a threshold-gated
// rescale, transposed products S^T = K Q^T and O^T += V^T P^T so that each
// lane owns one query column, K/V tiles streamed HBM -> LDS with
// global_load_lds (no VGPR staging), and the two-group ping-pong over each
// SIMD's wave pair.  The FP8 operands with fp32 accumulation follow
// "FlashAttention-3: Pipeline Assíncrono com Warp Specialization, WGMMA e FP8
// no Hopper e Blackwell", section "Estabilidade em FP8: Algoritmo de 2 Passos
// e Incoherent Processing" (E4M3: 1 sign, 4 exponent, 3 mantissa bits,
// range +-448).
//
// Products: v_mfma_f32_32x32x64_f8f6f4 (both operands e4m3).  Lane (m, h)
// of an operand holds 32 consecutive k-slots 32h .. 32h+31.
//  * S^T: A = K rows (32 bytes of one key row per lane, two ds_read_b128),
//    B = Q^T (32 bytes of the lane's query row, in VGPRs).
//  * P^T: lane-half h owns, in the S^T accumulators of a 64-key step, the
//    keys 8g + 4h + e (g = 0..7, e = 0..3); slot t = 4g + e of its B operand
//    holds key 8g + 4h + e, i.e. accumulator register t of block t/16 in
//    natural order.
//  * V^T: the A operand needs, per lane, 32 keys of one column.  Within each
//    64-key step V rows are stored in LDS under the key permutation
//        rho(8g + 4h + e) = 32h + 4g + e,
//    which makes a lane-half's 32 keys 32 consecutive LDS rows; the tile
//    loader applies it by choosing each lane's source row.  They are read
//    with four ds_read_b64_tr_b8 (transposing LDS reads: in each 16-lane
//    group, 8 rows x 16 columns, one column of 8 rows per lane).
// Scaling: x = code * descale[b,h].  Scores use c = |scale| log2(e) dq dk;
// probabilities are p' = exp2(s c - m_ref + P_OFFSET), at most
// 2^(TAU + P_OFFSET) = 256 < 448, rounded to e4m3 (RNE, v_cvt_pk_fp8_f32);
// the row sum l is accumulated from the fp32 p'; O = acc * dv / l, so the
// 2^P_OFFSET factor cancels; lse = ln2 * (m_ref - P_OFFSET + log2 l).
//
// Two-pass form (same section of the FA3 page: a first pass finds each row's
// exact maximum of the scores with fp32 accumulation, the second
// exponentiates and multiplies by V with static scale factors).  MODE 1
// runs only S^T = K Q^T and the row maximum m = max_j s_ij c over the
// visible keys, and stores m where lse goes; MODE 2 reads it back and runs
// the product with m fixed: no running maximum and no rescale, and
// p' = exp2(s c - m + 8) <= 2^8 for every key (the static scale 2^8 keeps
// p' inside e4m3's normal range down to p = 2^-14).  MODE 0 is the
// single-pass kernel.
#include <type_traits>

#include "attn_kernels.hpp"

namespace attn {

constexpr float kTauFp8 = 4.0f;
constexpr float kPOffset = 4.0f;   // kTauFp8 + kPOffset <= 8 keeps p' <= 256
constexpr float kPOffset2 = 8.0f;  // two-pass: the exact maximum gives p' <= 2^8

// 16-byte-chunk XOR swizzles of the row-major [BC][D]-byte LDS tiles (rows
// of D bytes; a 256-byte bank line spans 256/D rows).
//  K: 16 lanes read one chunk of 16 consecutive rows (ds_read_b128).
//  V: 32 lanes read 2 adjacent chunks of 8 consecutive rows (tr_b8).
template <int D> __device__ __forceinline__ int swz_k8(int row) {
  return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
template <int D> __device__ __forceinline__ int swz_v8(int row) {
  return D == 128 ? (((row >> 1) & 3) << 1) : (((row >> 2) & 1) << 1);
}
// tile key of LDS row r of a V tile (inverse of rho within each 64-key step)
__device__ __forceinline__ int v_row_key(int r) {
  return (r & ~63) + 8 * ((r >> 2) & 7) + 4 * ((r >> 5) & 1) + (r & 3);
}

__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d, int old) {
  // the untouched half of the first conversion's destination is written by
  // the second, so its old value may be anything: pass the dead word the
  // result replaces, so that the packs land in place
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D, int NW, int BC, bool CAUSAL, int MODE>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwd_fp8_kernel(FwdParams p) {
  static_assert(MODE >= 0 && MODE <= 2, "0 single pass, 1 row maximum, 2 fixed maximum");
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(BC == 64 || BC == 128, "kv tile");
  static_assert(NW == 8, "two groups of four waves, one wave of each per SIMD");
  constexpr int BR = NW * 32;            // query rows per work-group
  constexpr int NKB = BC / 32;           // 32-key blocks per tile
  constexpr int NKK = BC / 64;           // 64-key steps of the P.V product
  constexpr int NDB = D / 32;            // 32-wide column blocks of the output
  constexpr int NKS = D / 64;            // k-steps of the QK^T product
  constexpr int TILE = BC * D;           // bytes per K or V tile

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * TILE];
  unsigned char* ks_base = smem;         // K tiles: [2][BC][D]
  unsigned char* vs_base = smem + 2 * TILE;   // V tiles: [2][BC][D], rows permuted

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;             // 0: group A, 1: group B
  const int ln = lane & 31;
  const int lh = lane >> 5;

  // one work item (batch*head, query tile) per step; the loop runs once
  // unless the launch is persistent (never for the row-maximum pass, which
  // is compiled without the loop).  The item's first loads go into LDS
  // only after every wave has passed the previous item's last barrier.
  constexpr int kMaxSteps = MODE == 1 ? 1 : 0x7fffffff;
  for (int step = 0; step < kMaxSteps; ++step) {
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

  const unsigned char* __restrict__ qg = (const unsigned char*)p.q + sv.q_base;
  const unsigned char* __restrict__ kg = (const unsigned char*)p.k + sv.kv_base;
  const unsigned char* __restrict__ vg = (const unsigned char*)p.v + sv.kv_base;

  const float dq = p.dq[bh];
  const float dk = p.dk[b * p.Hkv + sv.hk];
  const float dv = p.dv[b * p.Hkv + sv.hk];
  // c = |scale dq dk| log2(e); a negative product flips the sign of Q
  float c = p.c * dq * dk;
  unsigned qsign = p.qsign;
  if (c < 0.f) {
    c = -c;
    qsign ^= 0x80808080u;
  }
  c = fmaxf(c, 1e-30f);
  // c is uniform over the work-group: in a scalar register, the softmax's
  // FMAs read two vector operands instead of three
  c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c)));

  // ---- Q^T fragments: lane (n=ln, h=lh) holds Q[myq][64ks + 32lh .. +31]
  i32x8 qf[NKS];
  {
    const int qr = myq < N ? myq : N - 1;
    const u32x4* src = (const u32x4*)(qg + (long long)qr * tok + 32 * lh);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 a = src[4 * ks] ^ qsign;
      u32x4 bq = src[4 * ks + 1] ^ qsign;
      i32x8 t;
      t[0] = a[0]; t[1] = a[1]; t[2] = a[2]; t[3] = a[3];
      t[4] = bq[0]; t[5] = bq[1]; t[6] = bq[2]; t[7] = bq[3];
      qf[ks] = t;
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

  // ---- tile loader (group A only, in its matrix-core phase, whose issue
  // slots are mostly free): global_load_lds_dwordx4 straight into
  // the LDS tile; lane l of a load fills bytes [16 l, 16 l + 16) after the
  // wave-uniform base (M0), so the K swizzle and the V row permutation are
  // applied by choosing each lane's source chunk.  Keys past N are clamped
  // to key N-1 (masked: p = 0 against finite V).
  constexpr int LPW = TILE / 1024 / 4;                   // loads per B wave per tensor per tile
  static_assert(LPW >= 1 && LPW * 1024 * 4 == TILE, "tile must split into 1 KiB per load");
  const int wb = wave & 3;
  int k_key[LPW], v_key[LPW];
  unsigned kgo[LPW], vgo[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int off = (wb * LPW + i) * 1024 + lane * 16;   // byte offset in the tile
    const int row = off / D;
    const int pc = (off - row * D) / 16;                  // physical 16-byte chunk
    const int vk = v_row_key(row);
    k_key[i] = row;
    v_key[i] = vk;
    // less 1024 (i % 4): the loads share M0 in groups of four (lds_dma_*);
    // still >= 0, as load i starts at least that many bytes into the tile
    kgo[i] = (unsigned)((long long)row * tkv + (pc ^ swz_k8<D>(row)) * 16) - (unsigned)((i & 3) * 1024);
    vgo[i] = (unsigned)((long long)vk * tkv + (pc ^ swz_v8<D>(row)) * 16) - (unsigned)((i & 3) * 1024);
  }
  const unsigned lds_k = (unsigned)(size_t)((ATTN_LDS unsigned char*)ks_base);
  const unsigned lds_v = (unsigned)(size_t)((ATTN_LDS unsigned char*)vs_base);
  const unsigned lds_wave = __builtin_amdgcn_readfirstlane((unsigned)(wb * LPW * 1024));
  // a tile's byte offset: one 32x32 -> 64-bit product of the tile index and
  // the tile's bytes (few scalar instructions in the loading phase); a full
  // tile: one compare against the count of full tiles
  const unsigned tile_bytes = (unsigned)BC * (unsigned)tkv;
  const int n_full = N / BC;
  auto load_tile = [&](const unsigned* go, const int* key, const unsigned char* src, unsigned lds_buf, int j) {
    const int kv0 = j * BC;
    const unsigned la0 = lds_buf + lds_wave;
    const unsigned char* base = src + (unsigned long long)(unsigned)j * tile_bytes;
    if (__builtin_expect(j < n_full, 1)) {
      lds_dma_tile_s<LPW>(la0, go, base);
    } else {
      const void* g[LPW];
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const long long back = (long long)(kv0 + key[i] < N ? 0 : kv0 + key[i] - (N - 1)) * tkv;
        g[i] = base + (long long)go[i] - back;
      }
      lds_dma_tile_v<LPW>(la0, g);
    }
  };
  auto load_k = [&](int j) { load_tile(kgo, k_key, kg, lds_k + (unsigned)((j & 1) * TILE), j); };
  auto load_v = [&](int j) { load_tile(vgo, v_key, vg, lds_v + (unsigned)((j & 1) * TILE), j); };
  auto wait_loads = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // ---- per-lane LDS read offsets (bytes)
  int koff[NKS][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int x = 0; x < 2; ++x)
      koff[ks][x] = ln * D + (((4 * ks + 2 * lh + x) ^ swz_k8<D>(ln)) * 16);
  const int gi = lane & 15;
  const int vrow_l = 32 * lh + (gi >> 1);                 // + 8u for the u-th read
  const int vsw = swz_v8<D>(vrow_l);                       // constant over u
  int voff[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int chunk = 2 * db + ((lane & 16) >> 4);
    voff[db] = vrow_l * D + ((chunk ^ vsw) * 16) + 8 * (gi & 1);
  }

  // ---- running state
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_ref = -__builtin_inff();
  if constexpr (MODE == 2) m_ref = p.lse[sv.lse_base + (myq < N ? myq : N - 1)];
  float l_part[4] = {0.f, 0.f, 0.f, 0.f};
  f32x16 s[NKB];
  i32x8 pf[NKK];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) pf[kk] = i32x8{};

  // ---- X_j: S^T of tile j+1 (K tile kt) and O^T += V_j^T P_j^T (V tile vt)
  auto phase_x = [&](auto qk_tag, auto pv_tag, const unsigned char* kt, const unsigned char* vt)
                     __attribute__((always_inline)) {
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr bool PV = decltype(pv_tag)::value;
    // the matrix-core phase issues first on its SIMD; the partner wave's
    // vector ALU work fills the remaining issue slots
    if constexpr (!PV) {
      // scores only (the first phase, and the row-maximum pass): left to the
      // compiler's schedule
      __builtin_amdgcn_s_setprio(3);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          u32x4 a0 = *(const u32x4*)(kt + kb * 32 * D + koff[ks][0]);
          u32x4 a1 = *(const u32x4*)(kt + kb * 32 * D + koff[ks][1]);
          i32x8 a;
          a[0] = a0[0]; a[1] = a0[1]; a[2] = a0[2]; a[3] = a0[3];
          a[4] = a1[0]; a[5] = a1[1]; a[6] = a1[2]; a[7] = a1[3];
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], ks == 0 ? f32x16{} : s[kb],
                                                                 0, 0, 0, 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      return;
    }
    // One stream of products, the S^T ones (ks-major, if QK) then the P.V
    // ones, each operand read from LDS PF products ahead of its MFMA (a
    // fence after every MFMA keeps that order whatever code surrounds the
    // phase).
    constexpr int PF = 2;
    constexpr int NQ = QK ? NKS * NKB : 0;
    constexpr int NP = NQ + NKK * NDB;
    i32x8 a[NP];
    auto rd = [&](int i) __attribute__((always_inline)) {
      i32x8 t;
      if (i < NQ) {
        const int ks = i / NKB, kb = i % NKB;
        const u32x4 a0 = *(const u32x4*)(kt + kb * 32 * D + koff[ks][0]);
        const u32x4 a1 = *(const u32x4*)(kt + kb * 32 * D + koff[ks][1]);
        t[0] = a0[0]; t[1] = a0[1]; t[2] = a0[2]; t[3] = a0[3];
        t[4] = a1[0]; t[5] = a1[1]; t[6] = a1[2]; t[7] = a1[3];
      } else {
        const int kk = (i - NQ) / NDB, db = (i - NQ) % NDB;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (ATTN_LDS i32x2*)(vt + kk * 64 * D + voff[db] + 8 * u * D));
          t[2 * u] = r[0];
          t[2 * u + 1] = r[1];
        }
      }
      a[i] = t;
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
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], qf[ks], ks == 0 ? f32x16{} : s[kb],
                                                               0, 0, 0, 0, 0, 0);
      } else {
        const int kk = (i - NQ) / NDB, db = (i - NQ) % NDB;
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], pf[kk], oacc[db], 0, 0, 0, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- Y_j: softmax of S_{j+1} (keys kv0 ..): mask, gated rescale of
  // m_ref / l / O, exponentials -> pf.
  //
  // Row maximum and gated rescale: m = max_j s_j c over the tile; where it
  // exceeds m_ref by more than TAU, m_ref moves to it and l and O are scaled
  // by exp2(m_ref_old - m), skipped by the whole wave when no row moved.
  // Afterwards every p' of the tile is at most 2^(TAU+P_OFFSET).  The
  // two-pass form's first pass keeps only the maximum.
  auto rescale = [&]() __attribute__((always_inline)) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[kb][r]), s[kb][r + 1]);
    mx = pair_max(mx);
    const float mt = mx * c;
    if constexpr (MODE == 1) {
      m_ref = fmaxf(m_ref, mt);
      return;
    }
    const bool need = mt > m_ref + kTauFp8;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? fast_exp2(m_ref - mt) : 1.f;
      m_ref = need ? mt : m_ref;
#pragma unroll
      for (int i = 0; i < 4; ++i) l_part[i] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
  };
  // p' = exp2(s c - m_ref + offset) of the tile, rounded to e4m3 into pf
  // (64-key step kk, slot t = 16 (kb & 1) + r; each pack lands in the P word
  // it replaces), and four partial row sums t of the fp32 p'.  One 32-key
  // block at a time: its FMAs, then its exponentials, then packs and sums,
  // so that no instruction waits on the one just before it.
  auto exponentials = [&](float* t, float offset) __attribute__((always_inline)) {
    const float bias = offset - m_ref;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 e;
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = __builtin_fmaf(s[kb][r], c, bias);
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = fast_exp2(e[r]);
      const int kk = kb >> 1, half = kb & 1;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        pf[kk][4 * half + g] =
            pack_fp8x4(e[4 * g], e[4 * g + 1], e[4 * g + 2], e[4 * g + 3], pf[kk][4 * half + g]);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (kb == 0 && r < 4)
          t[r] = e[r];
        else
          t[r & 3] += e[r];
      }
      // one block's p' live at a time: the scheduler does not interleave
      // the blocks
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto phase_y = [&](auto masked_tag, int kv0) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
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
    if constexpr (MODE == 1) {
      rescale();
      return;
    }
    // the two-pass form's second pass knows the exact row maximum: no
    // running maximum, no rescale
    if constexpr (MODE == 0) rescale();
    float t[4];
    exponentials(t, MODE == 2 ? kPOffset2 : kPOffset);
#pragma unroll
    for (int i = 0; i < 4; ++i) l_part[i] += t[i];
  };

  // ---- phase schedule ------------------------------------------------------
  // Group A runs X_j in phase 2j+2 and Y_j in phase 2j+3; group B one phase
  // later.  So K_t is read in phases 2t and 2t+1 and V_t in phases 2t+2 and
  // 2t+3 (from buffer t&1).  Group A loads K_{u+1} and V_u at the start of
  // its matrix-core phase 2u (into buffers last read in phases 2u-2 / 2u-1)
  // and waits for them at the end of phase 2u+1.  Every wave passes the same
  // number of phase barriers, 2 * wg_tiles + 2.
  //
  // A wave with T = wv_tiles tiles runs X_{-1} (S of tile 0 only), Y_{-1},
  // then X_j (both products; S only in the row-maximum pass) and Y_j for
  // j = 0 .. T-2, then X_{T-1} (P.V only), and idles to the last phase.
  // Only the wave's last tile can need the mask (the causal diagonal, a
  // ragged end), so the tiles before the first masked one run in a loop
  // without it.  The two groups run separate copies of the schedule, so
  // group A's loads and waits sit at fixed points of its phases.
  using T_ = std::true_type;
  using F_ = std::false_type;
  using PV_ = std::integral_constant<bool, MODE != 1>;
  const int n_phases = 2 * wg_tiles + 2;
  auto loads_for = [&](int u) {
    u = __builtin_amdgcn_readfirstlane(u);    // an SGPR for the loads' addresses
    if (u + 1 < wg_tiles) load_k(u + 1);
    if (MODE != 1 && u < wg_tiles) load_v(u);
  };
  auto kt_of = [&](int j) { return ks_base + ((j + 1) & 1) * TILE; };   // K tile of X_j
  auto vt_of = [&](int j) { return vs_base + (j & 1) * TILE; };         // V tile of X_j

  if (grp == 0 && wg_tiles > 0) load_k(0);
  wait_loads();
  __syncthreads();

  const int T = wv_tiles;
  // first tile that needs the mask: the causal diagonal or the ragged end
  int first_masked = N / BC;
  if (CAUSAL) first_masked = min(first_masked, (qw0 + 1) / BC);
  const int t_plain = min(first_masked, T);
  auto schedule = [&](auto loader_tag) __attribute__((always_inline)) {
    constexpr bool LOADER = decltype(loader_tag)::value;   // group A
    int ph = 0;
    // X phases start with group A's loads, Y phases end with its wait
    auto x_start = [&]() {
      if constexpr (LOADER) loads_for(ph >> 1);
    };
    auto y_end = [&]() {
      if constexpr (LOADER) wait_loads();
      __syncthreads();
      ++ph;
    };
    auto x_end = [&]() {
      __syncthreads();
      ++ph;
    };
    if constexpr (!LOADER) x_end();               // group B starts one phase later
    if (T > 0) {
      x_start();
      phase_x(T_{}, F_{}, kt_of(-1), vt_of(-1));
      x_end();
      if (first_masked <= 0)
        phase_y(T_{}, 0);
      else
        phase_y(F_{}, 0);
      y_end();
      int t = 1;
      for (; t < t_plain; ++t) {        // X_{t-1}, Y_{t-1} (softmax of tile t), unmasked
        x_start();
        phase_x(T_{}, PV_{}, kt_of(t - 1), vt_of(t - 1));
        x_end();
        phase_y(F_{}, t * BC);
        y_end();
      }
      for (; t < T; ++t) {              // the masked tail
        x_start();
        phase_x(T_{}, PV_{}, kt_of(t - 1), vt_of(t - 1));
        x_end();
        phase_y(T_{}, t * BC);
        y_end();
      }
      x_start();
      if constexpr (MODE != 1) phase_x(F_{}, T_{}, kt_of(T - 1), vt_of(T - 1));
      x_end();
    }
    // idle to the last phase (group A keeps loading for the other waves)
    for (; ph < n_phases;) {
      if (LOADER && (ph & 1) == 0) {
        x_start();
        x_end();
      } else {
        y_end();
      }
    }
  };
  if (grp == 0)
    schedule(T_{});
  else
    schedule(F_{});

  if constexpr (MODE == 1) {
    if (myq < N && lh == 0) p.lse[sv.lse_base + myq] = m_ref;
    continue;
  }
  // ---- epilogue: O = acc dv / l -> bf16, lse = ln2 (m_ref - offset + log2 l)
  const float l_tot = pair_sum((l_part[0] + l_part[1]) + (l_part[2] + l_part[3]));
  if (myq < N) {
    const float sc = dv / l_tot;
    __bf16* og = (__bf16*)p.o + sv.q_base + (long long)myq * tok;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * lh;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * g + 0] * sc, oacc[db][4 * g + 1] * sc);
        w[1] = pack_bf16x2(oacc[db][4 * g + 2] * sc, oacc[db][4 * g + 3] * sc);
        *(u32x2*)(og + d0) = w;
      }
    }
    if (lh == 0) {
      p.lse[sv.lse_base + myq] =
          (m_ref - (MODE == 2 ? kPOffset2 : kPOffset) + fast_log2(l_tot)) * 0.69314718055994531f;
    }
  }
  }   // work items
}

template <int D, int NW, int BC, bool CAUSAL>
static hipError_t launch_fp8_t(const FwdParams& prm, int grid, bool two_pass, hipStream_t stream) {
  if (!two_pass)
    return launch_kernel(attn_fwd_fp8_kernel<D, NW, BC, CAUSAL, 0>, dim3(grid), dim3(NW * 64),
                         stream, prm);
  // the row-maximum pass: one work-group per item (its items are short)
  FwdParams one = prm;
  one.persist = 0;
  const hipError_t e = launch_kernel(attn_fwd_fp8_kernel<D, NW, BC, CAUSAL, 1>, dim3(prm.items),
                                     dim3(NW * 64), stream, one);
  if (e != hipSuccess) return e;
  return launch_kernel(attn_fwd_fp8_kernel<D, NW, BC, CAUSAL, 2>, dim3(grid), dim3(NW * 64),
                       stream, prm);
}

// Waves per work-group: 8 (two per SIMD, one of each ping-pong group);
// keys per K/V tile: 128 (two 64-deep P.V steps), which halves the barriers
// per key of a 64-key tile and fits the register budget of the fp8 operands.
constexpr int kFp8Waves = 8;
constexpr int kFp8Tile = 128;

int fp8_rows_per_block(int d) { return kFp8Waves * 32; }

hipError_t launch_fp8(const FwdParams& prm, int d, int causal, int grid, bool two_pass,
                      hipStream_t stream) {
  if (d == 128) {
    return causal ? launch_fp8_t<128, kFp8Waves, kFp8Tile, true>(prm, grid, two_pass, stream)
                  : launch_fp8_t<128, kFp8Waves, kFp8Tile, false>(prm, grid, two_pass, stream);
  }
  return causal ? launch_fp8_t<64, kFp8Waves, kFp8Tile, true>(prm, grid, two_pass, stream)
                : launch_fp8_t<64, kFp8Waves, kFp8Tile, false>(prm, grid, two_pass, stream);
}

}  // namespace attn
