// OCP FP8 E4M3 tiled exact attention forward for gfx950 (MI355X, CDNA4).
//
// Same method and work decomposition as the bf16 kernel (attn_fwd_bf16.hip):
// online softmax over K/V tiles with a threshold-gated rescale, transposed
// products S^T = K Q^T and O^T += V^T P^T so each lane owns one query column.
// The FP8 operands with fp32 accumulation follow "FlashAttention-3: Pipeline
// Assíncrono com Warp Specialization, WGMMA e FP8 no Hopper e Blackwell",
// section "Estabilidade em FP8: Algoritmo de 2 Passos e Incoherent
// Processing" (E4M3: 1 sign, 4 exponent, 3 mantissa bits, range +-448).
//
// Products: v_mfma_f32_32x32x64_f8f6f4 (both operands e4m3).  Lane (m, h)
// of an operand holds 32 consecutive k-slots 32h .. 32h+31.
//  * S^T: A = K rows (32 bytes of one key row per lane, two ds_read_b128),
//    B = Q^T (32 bytes of the lane's query row, in VGPRs).
//  * P^T: lane-half h owns, in the S^T accumulators of a 64-key tile, the
//    keys 8g + 4h + e (g = 0..7, e = 0..3); slot t = 4g + e of its B operand
//    holds key 8g + 4h + e, i.e. accumulator register t of block t/16 in
//    natural order.
//  * V^T: the A operand needs, per lane, 32 keys of one column.  V rows are
//    therefore stored in LDS under the key permutation
//        rho(8g + 4h + e) = 32h + 4g + e,
//    which makes a lane-half's 32 keys 32 consecutive LDS rows, and are read
//    with four ds_read_b64_tr_b8 (transposing LDS reads: in each 16-lane
//    group, 8 rows x 16 columns, one column of 8 rows per lane).
// Scaling: x = code * descale[b,h].  Scores use c = |scale| log2(e) dq dk;
// probabilities are p' = exp2(s c - m_ref + P_OFFSET), at most
// 2^(TAU + P_OFFSET) = 256 < 448, rounded to e4m3 (RNE, v_cvt_pk_fp8_f32);
// the row sum l is accumulated from the fp32 p'; O = acc * dv / l, so the
// 2^P_OFFSET factor cancels; lse = ln2 * (m_ref - P_OFFSET + log2 l).
#include "attn_kernels.hpp"

namespace attn {

constexpr float kTauFp8 = 4.0f;
constexpr float kPOffset = 4.0f;   // kTauFp8 + kPOffset <= 8 keeps p' <= 256

// 16-byte-chunk XOR swizzles of the row-major [64][D]-byte LDS tiles (rows
// of D bytes; 16 chunks of a 256-byte bank line span 256/D rows).
//  K: 16 lanes read one chunk of 16 consecutive rows (ds_read_b128).
//  V: 32 lanes read 2 adjacent chunks of 8 consecutive rows (tr_b8).
template <int D> __device__ __forceinline__ int swz_k8(int row) {
  return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
template <int D> __device__ __forceinline__ int swz_v8(int row) {
  return D == 128 ? (((row >> 1) & 3) << 1) : (((row >> 2) & 1) << 1);
}
// LDS row of tile key kappa (0..63) in the V tile.
__device__ __forceinline__ int v_perm_row(int kappa) {
  return 32 * ((kappa >> 2) & 1) + 4 * (kappa >> 3) + (kappa & 3);
}

__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwd_fp8_kernel(FwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int BC = 64;                 // keys per tile (one 64-deep P.V product)
  constexpr int T = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int CPR = D / 16;            // 16-byte chunks per row
  constexpr int NCH = BC * CPR;          // chunks per tensor per tile
  constexpr int CPT = NCH >= T ? NCH / T : 1;
  static_assert(NCH >= T ? (CPT * T == NCH) : true, "tile must split evenly over threads");
  constexpr int NKB = BC / 32;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 64;

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * BC * D];
  unsigned char* ks_base = smem;
  unsigned char* vs_base = smem + 2 * BC * D;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31;
  const int lh = lane >> 5;

  int bh, qt;
  block_to_work(p, bh, qt);
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int N = p.N;
  const long long tok = (long long)p.H * D;
  const long long head_base = ((long long)b * N * p.H + h) * D;

  const int q0 = qt * BR;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + ln;

  const unsigned char* __restrict__ qg = (const unsigned char*)p.q + head_base;
  const unsigned char* __restrict__ kg = (const unsigned char*)p.k + head_base;
  const unsigned char* __restrict__ vg = (const unsigned char*)p.v + head_base;

  const float dq = p.dq[bh];
  const float dk = p.dk[bh];
  const float dv = p.dv[bh];
  const float c = p.c * dq * dk;

  // ---- Q^T fragments: lane (n=ln, h=lh) holds Q[myq][64ks + 32lh .. +31]
  i32x8 qf[NKS];
  {
    const int qr = myq < N ? myq : N - 1;
    const u32x4* src = (const u32x4*)(qg + (long long)qr * tok + 32 * lh);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 a = src[4 * ks] ^ p.qsign;
      u32x4 bq = src[4 * ks + 1] ^ p.qsign;
      i32x8 t;
      t[0] = a[0]; t[1] = a[1]; t[2] = a[2]; t[3] = a[3];
      t[4] = bq[0]; t[5] = bq[1]; t[6] = bq[2]; t[7] = bq[3];
      qf[ks] = t;
    }
  }

  const int n_kv_all = (N + BC - 1) / BC;
  int wg_tiles = n_kv_all;
  int wv_tiles = qw0 < N ? n_kv_all : 0;
  if (CAUSAL) {
    const int last_wg = min(q0 + BR - 1, N - 1);
    wg_tiles = last_wg / BC + 1;
    if (qw0 < N) wv_tiles = min(qw0 + 31, N - 1) / BC + 1;
  }

  // ---- cooperative loader
  u32x4 kreg[CPT], vreg[CPT];
  auto fetch = [&](int j) {
    const int kv0 = j * BC;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cc = tid + i * T;
      const int row = cc / CPR;
      const int col = cc - row * CPR;
      const int n = kv0 + row;
      if (cc < NCH && n < N) {
        const long long off = (long long)n * tok + col * 16;
        kreg[i] = *(const u32x4*)(kg + off);
        vreg[i] = *(const u32x4*)(vg + off);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto stash = [&](int buf) {
    unsigned char* kd = ks_base + buf * BC * D;
    unsigned char* vd = vs_base + buf * BC * D;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cc = tid + i * T;
      if (cc < NCH) {
        const int row = cc / CPR;
        const int col = cc - row * CPR;
        const int vrow = v_perm_row(row);
        *(u32x4*)(kd + row * D + ((col ^ swz_k8<D>(row)) * 16)) = kreg[i];
        *(u32x4*)(vd + vrow * D + ((col ^ swz_v8<D>(vrow)) * 16)) = vreg[i];
      }
    }
  };

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

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_ref = -__builtin_inff();
  float l_part = 0.f;

  if (wg_tiles > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();

  for (int j = 0; j < wg_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < wg_tiles) fetch(j + 1);

    if (j < wv_tiles) {
      const unsigned char* kt = ks_base + buf * BC * D;
      const unsigned char* vt = vs_base + buf * BC * D;
      const int kv0 = j * BC;

      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          u32x4 a0 = *(const u32x4*)(kt + kb * 32 * D + koff[ks][0]);
          u32x4 a1 = *(const u32x4*)(kt + kb * 32 * D + koff[ks][1]);
          i32x8 a;
          a[0] = a0[0]; a[1] = a0[1]; a[2] = a0[2]; a[3] = a0[3];
          a[4] = a1[0]; a[5] = a1[1]; a[6] = a1[2]; a[7] = a1[3];
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s[kb], 0, 0, 0, 0, 0, 0);
        }
      }

      const bool masked = (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0);
      unsigned vis = ~0u;
      float mx = -__builtin_inff();
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            const bool ok = key < N && (!CAUSAL || key <= myq);
            if (!ok) vis &= ~(1u << (kb * 16 + r));
            mx = fmaxf(mx, ok ? s[kb][r] : -__builtin_inff());
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
      mx = pair_max(mx);

      const float mt = mx * c;
      const bool need = mt > m_ref + kTauFp8;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? fast_exp2(m_ref - mt) : 1.f;
        m_ref = need ? mt : m_ref;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }

      // p' = exp2(s c - m_ref + P_OFFSET); slot t = 16 kb + r
      const float bias = kPOffset - m_ref;
      i32x8 pf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float e[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = 4 * w + x;
            float y = fast_exp2(__builtin_fmaf(s[kb][r], c, bias));
            if (masked) y = ((vis >> (kb * 16 + r)) & 1u) ? y : 0.f;
            e[x] = y;
            l_part += y;
          }
          pf[kb * 4 + w] = pack_fp8x4(e[0], e[1], e[2], e[3]);
        }
      }

      // O^T += V_j^T P^T
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        i32x8 a;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (ATTN_LDS i32x2*)(vt + voff[db] + 8 * u * D));
          a[2 * u] = t[0];
          a[2 * u + 1] = t[1];
        }
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, oacc[db], 0, 0, 0, 0, 0, 0);
      }
    }

    if (j + 1 < wg_tiles) stash(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = pair_sum(l_part);
  if (myq < N) {
    const float sc = dv / l_tot;
    __bf16* og = (__bf16*)p.o + head_base + (long long)myq * tok;
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
      p.lse[(long long)bh * N + myq] =
          (m_ref - kPOffset + fast_log2(l_tot)) * 0.69314718055994531f;
    }
  }
}

template <int D, int NW, bool CAUSAL>
static hipError_t launch_fp8_t(const FwdParams& prm, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, NW, CAUSAL>), dim3(grid), dim3(NW * 64), 0, stream,
                     prm);
  return hipGetLastError();
}

int fp8_rows_per_block(int d) { return (d == 128 ? 8 : 8) * 32; }

hipError_t launch_fp8(const FwdParams& prm, int d, int causal, int grid, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch_fp8_t<128, 8, true>(prm, grid, stream)
                  : launch_fp8_t<128, 8, false>(prm, grid, stream);
  }
  return causal ? launch_fp8_t<64, 8, true>(prm, grid, stream)
                : launch_fp8_t<64, 8, false>(prm, grid, stream);
}

}  // namespace attn
