// bf16 backward of the tiled exact attention for gfx950 (MI355X, CDNA4).
//
// Gradients of O = softmax(Q K^T * scale) V with respect to Q, K and V (the
// backward pass that "FlashAttention 4: Atenção Mais Rápida e Eficiente em
// Memória para LLMs", section "Principais Conclusões", and "FlashAttention-4
// no Blackwell B200 ...", section "Redução de tráfego no backward", name as
// the forward kernel's counterpart), by the chain rule on the definition:
//   P = softmax(scale Q K^T)  (recomputed tile by tile from the forward's
//                              log-sum-exp: P = exp2(scale log2(e) S - lse log2(e)))
//   dV = P^T dO,   dP = dO V^T,   D_i = sum_c dO_ic O_ic,
//   dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q.
// Like the forward, the N x N matrices P, dP, dS never reach HBM.
//
// Three kernels (four at d = 128), enqueued in order on the caller's stream:
//   delta : D_i for every row (a dot product of two rows), into the caller's
//           fp32 workspace [B][H][N];
//   dQ    : one work-group per (batch, head, 256 queries); each wave owns 32
//           query columns and streams 64-key K/V tiles through LDS:
//             S^T = K Q^T, dP^T = V dO^T (A = K / V rows, B = Q^T / dO^T in
//             VGPRs), dS^T = P^T (dP^T - D), dQ^T += K^T dS^T (A = K^T from
//             transposing LDS reads, B = dS^T packed to bf16);
//   dK/dV : one work-group per (batch, head, 256 keys); each wave owns 32
//           key columns (its K and V rows in registers; at d = 128 dV and dK
//           come from two kernels, see below) and streams 64-query Q / dO
//           tiles (plus their lse and D values) through LDS:
//             S = Q K^T, dP = dO V^T (A = Q / dO rows), dS = P (dP - D),
//             dV^T += dO^T P, dK^T += Q^T dS (A = dO^T / Q^T from transposing
//             LDS reads, B = P / dS packed to bf16).
// No atomics: each output element is produced by exactly one lane, so the
// results are deterministic.  The lane ownership, the 32x32x16 bf16 MFMA
// layouts and the key/query permutation of the packed operands are those of
// the forward kernel (attn_fwd_bf16.hip); masked entries get P = 0 after the
// exponential, so the scale may have either sign.
#include <type_traits>

#include "attn_kernels.hpp"

namespace attn {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  int B, H, N;
  int n_tiles;       // ceil(N / 256): query tiles per head (dQ)
  int n_ktiles;      // ceil(N / 256): key tiles per head (dK/dV)
  int tile_major;    // 1: tile-major block order (see bwd_work)
  float c;           // scale * log2(e)
  float scale;
};

constexpr float kLog2e = 1.4426950408889634f;

// 16-byte-chunk XOR swizzle of the row-major [rows][D] LDS tiles, read
// two ways: a ds_read_b128 of 16 lanes takes one chunk of 16 consecutive
// rows, so the swizzle must be a bijection over them (over the 8 rows of
// one parity at D = 64, where a 256-byte bank line holds two rows); a
// transposing read takes 4 consecutive chunks of 8 consecutive rows, so the
// swizzle's high bits must put those rows' chunk groups on all four 64-byte
// quarters of the bank line, twice each.  Both reads are then free of bank
// conflicts.
template <int D> __device__ __forceinline__ int swz_b(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  const int k = (row >> 1) & 7;
  return k ^ ((k & 1) << 2);
}

__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
  return __uint_as_float((unsigned)b << 16);
}

// ---------------------------------------------------------------------------
// delta: D[b][h][n] = sum_c dO[b][n][h][c] O[b][n][h][c]; 16 lanes per row
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(BwdParams p) {
  constexpr int LPR = 16;                 // lanes per row
  constexpr int EPL = D / LPR;            // elements per lane (8 or 4)
  const long long rows = (long long)p.B * p.N * p.H;
  const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const unsigned short* o = (const unsigned short*)p.o + row * D + sub * EPL;
    const unsigned short* g = (const unsigned short*)p.dout + row * D + sub * EPL;
    unsigned short ob[EPL], gb[EPL];
    if constexpr (EPL == 8) {
      *(u32x4*)ob = *(const u32x4*)o;
      *(u32x4*)gb = *(const u32x4*)g;
    } else {
      *(u32x2*)ob = *(const u32x2*)o;
      *(u32x2*)gb = *(const u32x2*)g;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = __builtin_fmaf(bf16_to_f32(ob[e]), bf16_to_f32(gb[e]), acc);
  }
  acc += __shfl_xor(acc, 8, LPR);
  acc += __shfl_xor(acc, 4, LPR);
  acc += __shfl_xor(acc, 2, LPR);
  acc += __shfl_xor(acc, 1, LPR);
  if (sub == 0 && row < rows) {
    const long long nh = (long long)p.N * p.H;
    const long long b = row / nh;
    const long long rem = row - b * nh;
    const long long n = rem / p.H;
    const long long h = rem - n * p.H;
    p.delta[(b * p.H + h) * p.N + n] = acc;
  }
}

// Tile loader shared by the dQ and dK/dV kernels: NW waves each fill LPW
// 1 KiB pieces of a [ROWS][D] bf16 tile with
// global_load_lds_dwordx4 (lane l fills bytes [16 l, 16 l + 16) after the
// wave-uniform base in M0), choosing each lane's source chunk so that the
// tile lands swizzled; rows past N are clamped to row N-1.
template <int D, int NW, int ROWS = 64>
struct TileLoader {
  static constexpr int TILE = ROWS * D;
  static constexpr int LPW = TILE * 2 / 1024 / NW;
  static_assert(LPW >= 1 && LPW * 1024 * NW == TILE * 2, "tile must split into 1 KiB per load");
  int row[LPW];
  unsigned go[LPW];
  unsigned lds_wave;
  __device__ void init(int wave, int lane, long long tok) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int off = (wave * LPW + i) * 512 + lane * 8;   // element offset in the tile
      const int r = off / D;
      const int pc = (off - r * D) / 8;
      row[i] = r;
      go[i] = (unsigned)(((long long)r * tok + (pc ^ swz_b<D>(r)) * 8) * 2);
    }
    lds_wave = __builtin_amdgcn_readfirstlane((unsigned)(wave * LPW * 1024));
  }
  // rows row0 .. row0+ROWS-1 of the tensor at src (element (row, 0) = src + row*tok)
  __device__ void load(const __bf16* src, long long tok, unsigned lds_buf, int row0, int N) const {
    const unsigned la0 = lds_buf + lds_wave;
    const __bf16* base = src + (long long)row0 * tok;
    if (row0 + ROWS <= N) {
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(la0 + i * 1024),
                     "v"(go[i]), "s"(base)
                     : "memory");
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const long long back = (long long)(row0 + row[i] < N ? 0 : row0 + row[i] - (N - 1)) * tok;
        const __bf16* g = base + (long long)(go[i] / 2) - back;
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(la0 + i * 1024),
                     "v"(g)
                     : "memory");
      }
    }
  }
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Work-group -> (head, tile) order that keeps each head on one XCD: the
// hardware deals consecutive work-groups round-robin to the 8 XCDs (each
// with its own L2), so work-group L runs on XCD L % 8; giving XCD x the
// contiguous logical range [x G/8, (x+1) G/8) puts all tiles of a head on
// one L2, which then serves the K/V (or Q/dO) tiles every work-group of
// that head streams.
__device__ __forceinline__ int xcd_order(int L) {
  const int total = gridDim.x;
  if ((total & 7) != 0) return L;
  return (L & 7) * (total >> 3) + (L >> 3);
}

// (batch*head, rank) of work-group L for n tiles per head; rank 0 is the
// head's longest tile.  Head-major within each XCD (xcd_order), except for
// causal calls with few tiles per head (tile_major, B*H divisible by 8):
// their causal tile lengths do not pair up over an XCD's 32 CUs, so each XCD
// keeps its share of the heads but runs the longest tile of every head
// first, then the next longest.
__device__ __forceinline__ void bwd_work(const BwdParams& p, int n, int& bh, int& rank) {
  const int L = blockIdx.x;
  if (p.tile_major) {
    const int hx = (p.B * p.H) >> 3;
    const int k = L >> 3;
    rank = k / hx;
    bh = (L & 7) * hx + (k - rank * hx);
    return;
  }
  const int Lx = xcd_order(L);
  bh = Lx / n;
  rank = Lx - bh * n;
}

// Ordinary global loads issued before the tile loop must complete before
// it: the compiler's own wait for a value loaded earlier counts every
// outstanding vector-memory load, the direct-to-LDS tile loads included,
// so a first use inside the loop would wait for the next tile as well.
// An empty asm that reads the registers moves that wait here.
template <typename T>
__device__ __forceinline__ void loaded(const T& x) {
  asm volatile("" ::"v"(x));
}

// Per-lane element offsets of the transposing reads of a swizzled [rows][D]
// tile that give a lane (m = ln of a 32-wide column block db, h = lh) the
// 8 rows 4h + (t&3) + 8(t>>2) (t = 0..7) of a 16-row group: the low 4 rows
// from `lo`, the high 4 from `hi` (the swizzle differs between them).
template <int D, int NDB>
struct TrOffsets {
  int lo[NDB], hi[NDB];
  __device__ void init(int lane) {
    const int gi = lane & 15;
    const int lh = lane >> 5;
    const int r_lo = 4 * lh + (gi >> 2);
    const int r_hi = r_lo + 8;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int chunk = 4 * db + ((lane & 16) >> 3) + ((gi & 3) >> 1);
      lo[db] = r_lo * D + ((chunk ^ swz_b<D>(r_lo)) * 8) + (gi & 1) * 4;
      hi[db] = r_hi * D + ((chunk ^ swz_b<D>(r_hi)) * 8) + (gi & 1) * 4;
    }
  }
};

// A operand from two transposing reads (rows 16-row group at `base`)
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* base, int lo, int hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(base + lo));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(base + hi));
  const u32x2 a2 = __builtin_bit_cast(u32x2, a);
  const u32x2 b2 = __builtin_bit_cast(u32x2, b);
  u32x4 w;
  w[0] = a2[0];
  w[1] = a2[1];
  w[2] = b2[0];
  w[3] = b2[1];
  return __builtin_bit_cast(bf16x8, w);
}

// bf16 [row][D] store of a 32x32 accumulator block set (lane owns row `row`,
// register 4g+x of block db holds column 32 db + 8 g + 4 lh + x), scaled
template <int NDB>
__device__ __forceinline__ void store_rows(__bf16* dst, const f32x16 (&acc)[NDB], float s, int lh) {
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * lh;
      u32x2 w;
      w[0] = pack_bf16x2(acc[db][4 * g + 0] * s, acc[db][4 * g + 1] * s);
      w[1] = pack_bf16x2(acc[db][4 * g + 2] * s, acc[db][4 * g + 3] * s);
      *(u32x2*)(dst + d0) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: per (batch, head, 256 query rows); 64-key K/V tiles
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_kernel(BwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int BR = 256, BC = 64;
  constexpr int NKB = BC / 32, NKK = BC / 16, NKS = D / 16, NDB = D / 32;
  constexpr int TILE = BC * D;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * TILE];
  __bf16* ks_base = smem;
  __bf16* vs_base = smem + 2 * TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31;
  const int lh = lane >> 5;

  int bh, rank;
  bwd_work(p, p.n_tiles, bh, rank);
  const int qt = p.n_tiles - 1 - rank;   // longest first
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int N = p.N;
  const long long tok = (long long)p.H * D;
  const long long head_base = ((long long)b * N * p.H + h) * D;
  const int q0 = qt * BR;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + ln;
  const int qr = myq < N ? myq : N - 1;

  const __bf16* __restrict__ qg = (const __bf16*)p.q + head_base;
  const __bf16* __restrict__ kg = (const __bf16*)p.k + head_base;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + head_base;
  const __bf16* __restrict__ gg = (const __bf16*)p.dout + head_base;

  // Q^T and dO^T fragments (B operands): lane (n = ln, h = lh) holds row
  // myq, columns 16 ks + 8 lh .. +7
  bf16x8 qf[NKS], gf[NKS];
  {
    const u32x4* qs = (const u32x4*)(qg + (long long)qr * tok + 8 * lh);
    const u32x4* gs = (const u32x4*)(gg + (long long)qr * tok + 8 * lh);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, qs[2 * ks]);
      gf[ks] = __builtin_bit_cast(bf16x8, gs[2 * ks]);
    }
  }
  const float lse2 = p.lse[(long long)bh * N + qr] * kLog2e;
  const float dd = p.delta[(long long)bh * N + qr];
  const float c = p.c;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    loaded(qf[ks]);
    loaded(gf[ks]);
  }
  loaded(lse2);
  loaded(dd);

  const int n_kv_all = (N + BC - 1) / BC;
  int wg_tiles = n_kv_all;
  int wv_tiles = qw0 < N ? n_kv_all : 0;
  if (CAUSAL) {
    wg_tiles = min(q0 + BR - 1, N - 1) / BC + 1;
    if (qw0 < N) wv_tiles = min(qw0 + 31, N - 1) / BC + 1;
  }

  TileLoader<D, 8> ld;
  ld.init(wave, lane, tok);
  const unsigned lds_k = (unsigned)(size_t)((ATTN_LDS __bf16*)ks_base);
  const unsigned lds_v = (unsigned)(size_t)((ATTN_LDS __bf16*)vs_base);

  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = ln * D + (((2 * ks + lh) ^ swz_b<D>(ln)) * 8);
  TrOffsets<D, NDB> tro;
  tro.init(lane);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  if (wg_tiles > 0) {
    ld.load(kg, tok, lds_k, 0, N);
    ld.load(vg, tok, lds_v, 0, N);
  }
  wait_vmem();
  __syncthreads();

  // one K/V tile of this wave: S^T and dP^T, dS^T, dQ^T += K^T dS^T
  // buf_tag: the buffer of tile j (j & 1) when known at compile time
  // (0 or 1: the LDS addresses fold into the reads' offsets), else -1
  auto tile = [&](auto masked_tag, auto buf_tag, int j) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value;
    const int buf = BUF < 0 ? (j & 1) : BUF;
    const __bf16* kt = ks_base + buf * TILE;
    const __bf16* vt = vs_base + buf * TILE;
    const int kv0 = j * BC;
    f32x16 s[NKB], dp[NKB];
    // the matrix-core sections raise the wave's issue priority, so that
    // the partner wave's vector work fills the slots around its MFMAs
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 ka = *(const bf16x8*)(kt + kb * 32 * D + koff[ks]);
        const bf16x8 va = *(const bf16x8*)(vt + kb * 32 * D + koff[ks]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], ks == 0 ? f32x16{} : s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[ks], ks == 0 ? f32x16{} : dp[kb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // key kv0 + off (off = kb*32 + 8*(r/4) + 4*lh + r%4) is visible iff off - 4*lh <= lim
    const int lim = min(CAUSAL ? myq - kv0 - 4 * lh : 0x7fffffff, N - 1 - kv0 - 4 * lh);
    bf16x8 dsf[NKK];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = half * 8 + 2 * t;
          float p0 = fast_exp2(__builtin_fmaf(s[kb][r], c, -lse2));
          float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], c, -lse2));
          if constexpr (MASKED) {
            if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) p0 = 0.f;
            if (kb * 32 + 8 * ((r + 1) >> 2) + ((r + 1) & 3) > lim) p1 = 0.f;
          }
          w[t] = pack_bf16x2(p0 * (dp[kb][r] - dd), p1 * (dp[kb][r + 1] - dd));
        }
        dsf[kb * 2 + half] = __builtin_bit_cast(bf16x8, w);
      }
    }
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 a = tr_operand(kt + kk * 16 * D, tro.lo[db], tro.hi[db]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsf[kk], acc[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // the next tile's loads (every wave takes part), then this tile
  auto next_loads = [&](int j) __attribute__((always_inline)) {
    j = __builtin_amdgcn_readfirstlane(j);    // every wave counts the same tiles; SGPR addresses
    if (j + 1 < wg_tiles) {
      const unsigned nb = (unsigned)(((j + 1) & 1) * TILE * 2);
      ld.load(kg, tok, lds_k + nb, (j + 1) * BC, N);
      ld.load(vg, tok, lds_v + nb, (j + 1) * BC, N);
    }
  };
  auto end_tile = [&]() __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
  };
  // Only the wave's last tile can need the mask (the causal diagonal, a
  // ragged end): the tiles before the first masked one run without it.
  int first_masked = N / BC;
  if (CAUSAL) first_masked = min(first_masked, (qw0 + 1) / BC);
  using T_ = std::true_type;
  using F_ = std::false_type;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using BRT = std::integral_constant<int, -1>;
  int j = 0;
  const int j_plain = min(first_masked, wv_tiles);
  for (; j + 1 < j_plain; j += 2) {     // unmasked, two tiles per step (j even)
    next_loads(j);
    tile(F_{}, B0{}, j);
    end_tile();
    next_loads(j + 1);
    tile(F_{}, B1{}, j + 1);
    end_tile();
  }
  for (; j < j_plain; ++j) {
    next_loads(j);
    tile(F_{}, BRT{}, j);
    end_tile();
  }
  for (; j < wv_tiles; ++j) {
    next_loads(j);
    tile(T_{}, BRT{}, j);
    end_tile();
  }
  for (; j < wg_tiles; ++j) {           // the other waves' tiles: loads and barriers only
    next_loads(j);
    end_tile();
  }

  if (myq < N) store_rows<NDB>((__bf16*)p.dq + head_base + (long long)myq * tok, acc, p.scale, lh);
}

// ---------------------------------------------------------------------------
// dK / dV: per (batch, head, 256 key rows); 64-query Q / dO tiles.  Each of
// the 8 waves (two per SIMD) owns 32 keys.  At D = 64 one kernel produces
// both gradients (WANT = 3).  At D = 128 the K and V rows of a wave and two
// 32 x 128 fp32 accumulators do not fit the 256 registers of a wave that
// shares its SIMD, so two kernels run instead: dV (WANT = 1: S, P, dV^T) and
// dK (WANT = 2: S, P, dP, dS, dK^T), which recompute S.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int WANT>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(WANT >= 1 && WANT <= 3, "dV (1), dK (2) or both (3)");
  constexpr bool DV = (WANT & 1) != 0;
  constexpr bool DK = (WANT & 2) != 0;
  constexpr int NW = 8;
  constexpr int BK = NW * 32, BQ = 64;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int TILE = BQ * D;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * TILE];
  __shared__ __attribute__((aligned(16))) float rowv[2][2][BQ];   // [buffer][lse2, D][query]
  __bf16* qs_base = smem;
  __bf16* gs_base = smem + 2 * TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31;
  const int lh = lane >> 5;

  int bh, kt;
  bwd_work(p, p.n_ktiles, bh, kt);      // causal: low key tiles see the most queries
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int N = p.N;
  const long long tok = (long long)p.H * D;
  const long long head_base = ((long long)b * N * p.H + h) * D;
  const int k0 = kt * BK;
  const int kw0 = k0 + wave * 32;
  const int mykey = kw0 + ln;
  const int kr = mykey < N ? mykey : N - 1;

  const __bf16* __restrict__ qg = (const __bf16*)p.q + head_base;
  const __bf16* __restrict__ kg = (const __bf16*)p.k + head_base;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + head_base;
  const __bf16* __restrict__ gg = (const __bf16*)p.dout + head_base;

  // K^T and V^T fragments (B operands of S = Q K^T and dP = dO V^T): lane
  // (n = ln, h = lh) holds row mykey, columns 16 ks + 8 lh .. +7
  bf16x8 kf[NKS], vf[DK ? NKS : 1];
  {
    const u32x4* ks = (const u32x4*)(kg + (long long)kr * tok + 8 * lh);
    const u32x4* vs = (const u32x4*)(vg + (long long)kr * tok + 8 * lh);
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      kf[i] = __builtin_bit_cast(bf16x8, ks[2 * i]);
      if constexpr (DK) vf[i] = __builtin_bit_cast(bf16x8, vs[2 * i]);
    }
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      loaded(kf[i]);
      if constexpr (DK) loaded(vf[i]);
    }
  }
  const float c = p.c;

  const int n_q_all = (N + BQ - 1) / BQ;
  const int first = CAUSAL ? k0 / BQ : 0;

  TileLoader<D, NW> ld;
  ld.init(wave, lane, tok);
  const unsigned lds_q = (unsigned)(size_t)((ATTN_LDS __bf16*)qs_base);
  const unsigned lds_g = (unsigned)(size_t)((ATTN_LDS __bf16*)gs_base);
  const float* __restrict__ lse_h = p.lse + (long long)bh * N;
  const float* __restrict__ del_h = p.delta + (long long)bh * N;
  // lse (log2 units) and D of the tile's 64 query rows, by wave 0: loaded
  // with the tile, written to LDS once the tile's loads have completed
  float row_lse = 0.f, row_del = 0.f;
  auto load_rows = [&](int qt0) {
    if (wave == 0) {
      const int r = min(qt0 + lane, N - 1);
      row_lse = lse_h[r];
      row_del = del_h[r];
    }
  };
  auto store_rows_lds = [&](int buf) {
    if (wave == 0) {
      rowv[buf][0][lane] = row_lse * kLog2e;
      rowv[buf][1][lane] = row_del;
    }
  };

  int qoff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qoff[ks] = ln * D + (((2 * ks + lh) ^ swz_b<D>(ln)) * 8);
  TrOffsets<D, NDB> tro;
  tro.init(lane);

  f32x16 dk[DK ? NDB : 1], dv[DV ? NDB : 1];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    if constexpr (DK) dk[db] = f32x16{};
    if constexpr (DV) dv[db] = f32x16{};
  }

  if (first < n_q_all) {
    ld.load(qg, tok, lds_q, first * BQ, N);
    ld.load(gg, tok, lds_g, first * BQ, N);
    load_rows(first * BQ);
  }
  wait_vmem();
  if (first < n_q_all) store_rows_lds(0);
  __syncthreads();

  // one query tile j of this wave's keys
  // buf_tag: the buffer of tile j ((j - first) & 1) when known at compile
  // time (0 or 1: the LDS addresses fold into the reads' offsets), else -1
  auto tile = [&](auto masked_tag, auto buf_tag, int j) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value;
    const int buf = BUF < 0 ? ((j - first) & 1) : BUF;
    const int qt0 = j * BQ;
    const __bf16* qt = qs_base + buf * TILE;
    const __bf16* gt = gs_base + buf * TILE;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 qa = *(const bf16x8*)(qt + qb * 32 * D + qoff[ks]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
        if constexpr (DK) {
          const bf16x8 ga = *(const bf16x8*)(gt + qb * 32 * D + qoff[ks]);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[ks], dp, 0, 0, 0);
        }
      }
      // register r holds query qt0 + 32 qb + 8 (r/4) + 4 lh + r%4 of key mykey
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        u32x4 wp, wd;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int rb = 8 * g + 4 * half;                        // registers rb .. rb+3
          const int qi = 32 * qb + 8 * (rb >> 2) + 4 * lh;        // their first tile row
          const f32x4 lv = *(const f32x4*)&rowv[buf][0][qi];
          const f32x4 dv4 = *(const f32x4*)&rowv[buf][1][qi];
          float pv[4], dsv[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            float pe = fast_exp2(__builtin_fmaf(s[rb + x], c, -lv[x]));
            if constexpr (MASKED) {
              const int q = qt0 + qi + x;
              if (q >= N || (CAUSAL && mykey > q)) pe = 0.f;
            }
            pv[x] = pe;
            dsv[x] = pe * (dp[rb + x] - dv4[x]);
          }
          wp[2 * half] = pack_bf16x2(pv[0], pv[1]);
          wp[2 * half + 1] = pack_bf16x2(pv[2], pv[3]);
          wd[2 * half] = pack_bf16x2(dsv[0], dsv[1]);
          wd[2 * half + 1] = pack_bf16x2(dsv[2], dsv[3]);
        }
        pf[g] = __builtin_bit_cast(bf16x8, wp);
        dsf[g] = __builtin_bit_cast(bf16x8, wd);
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int rowb = (32 * qb + 16 * g) * D;
          if constexpr (DV) {
            const bf16x8 ga = tr_operand(gt + rowb, tro.lo[db], tro.hi[db]);
            dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, pf[g], dv[db], 0, 0, 0);
          }
          if constexpr (DK) {
            const bf16x8 qa = tr_operand(qt + rowb, tro.lo[db], tro.hi[db]);
            dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dsf[g], dk[db], 0, 0, 0);
          }
        }
      }
    }
  };
  // the next tile's loads (every wave takes part) ...
  auto next_loads = [&](int j) __attribute__((always_inline)) {
    j = __builtin_amdgcn_readfirstlane(j);    // every wave counts the same tiles; SGPR addresses
    if (j + 1 < n_q_all) {
      const unsigned nb = (unsigned)((((j - first) & 1) ^ 1) * TILE * 2);
      ld.load(qg, tok, lds_q + nb, (j + 1) * BQ, N);
      ld.load(gg, tok, lds_g + nb, (j + 1) * BQ, N);
      load_rows((j + 1) * BQ);
    }
  };
  // ... and after the tile, their row values into LDS and the barrier
  auto end_tile = [&](int j) __attribute__((always_inline)) {
    wait_vmem();
    if (j + 1 < n_q_all) store_rows_lds(((j - first) & 1) ^ 1);
    __syncthreads();
  };
  // Query tiles of this wave's keys, in order: inactive (all queries
  // precede the keys, causal), masked (the causal diagonal), unmasked,
  // masked (the ragged end).  The masked test the tiles had, by tile:
  // (qt0 + BQ > N) or (causal and qt0 < kw0 + 31); active iff kw0 < N and
  // (not causal or qt0 + BQ - 1 >= kw0).
  const int n = n_q_all;
  const int j_act = kw0 >= N ? n : (CAUSAL ? max(first, kw0 / BQ) : first);
  const int j_um = CAUSAL ? max(j_act, (kw0 + 31 + BQ - 1) / BQ) : j_act;
  const int seg_b = max(j_act, min(j_um, n));
  const int seg_c = max(seg_b, min(N / BQ, n));
  using T_ = std::true_type;
  using F_ = std::false_type;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using BRT = std::integral_constant<int, -1>;
  int j = first;
  for (; j < min(j_act, n); ++j) {      // inactive: loads and barriers only
    next_loads(j);
    end_tile(j);
  }
  for (; j < seg_b; ++j) {
    next_loads(j);
    tile(T_{}, BRT{}, j);
    end_tile(j);
  }
  // unmasked: two tiles per step from an even (j - first), so that the
  // buffers of each step are known at compile time
  if (j < seg_c && ((j - first) & 1)) {
    next_loads(j);
    tile(F_{}, BRT{}, j);
    end_tile(j);
    ++j;
  }
  for (; j + 1 < seg_c; j += 2) {
    next_loads(j);
    tile(F_{}, B0{}, j);
    end_tile(j);
    next_loads(j + 1);
    tile(F_{}, B1{}, j + 1);
    end_tile(j + 1);
  }
  for (; j < seg_c; ++j) {
    next_loads(j);
    tile(F_{}, BRT{}, j);
    end_tile(j);
  }
  for (; j < n; ++j) {
    next_loads(j);
    tile(T_{}, BRT{}, j);
    end_tile(j);
  }

  if (mykey < N) {
    if constexpr (DK) store_rows<NDB>((__bf16*)p.dk + head_base + (long long)mykey * tok, dk, p.scale, lh);
    if constexpr (DV) store_rows<NDB>((__bf16*)p.dv + head_base + (long long)mykey * tok, dv, 1.f, lh);
  }
}

// ---------------------------------------------------------------------------
// dK / dV in the forward's two-group ping-pong, per (batch, head, 256 key
// rows) with Q / dO tiles of BQ queries; the wave ownership and products are
// those of attn_bwd_dkdv_kernel above.  Launched for the dV kernel at
// D = 128 (WANT = 1, BQ = 64), where it is ~10% faster than the sequential
// form; for dK (more registers: a 64-query tile spills) and at D = 64 the
// sequential form is faster.  Waves 0-3 (group A) and 4-7 (group B, one
// phase behind) alternate
//   X_j (matrix cores): dV^T += dO_j^T P_j and / or dK^T += Q_j^T dS_j, then
//                       S (and dP) of tile j+1;
//   Y_j (vector ALU):   P (and dS) of tile j+1.
// A tile is read in four phases (its S / dP, then its update), so Q and dO
// tiles rotate through three LDS buffers, as do the tiles' lse and D values;
// group A issues the loads of tile u+1 at the start of its matrix-core phase
// 2u and waits for them at the end of phase 2u+1, when wave 0 also writes
// the lse and D values to LDS.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int WANT, int BQ>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_pp_kernel(BwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(WANT >= 1 && WANT <= 3, "dV (1), dK (2) or both (3)");
  static_assert(BQ == 32 || BQ == 64, "query tile");
  constexpr bool DV = (WANT & 1) != 0;
  constexpr bool DK = (WANT & 2) != 0;
  constexpr int NW = 8;
  constexpr int BK = NW * 32;
  constexpr int NQB = BQ / 32;           // 32-query blocks per tile
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int TILE = BQ * D;
  __shared__ __attribute__((aligned(16))) __bf16 smem[6 * TILE];
  __shared__ __attribute__((aligned(16))) float rowv[3][2][BQ];   // [buffer][lse2, D][query]
  __bf16* qs_base = smem;                // Q tiles:  [3][BQ][D]
  __bf16* gs_base = smem + 3 * TILE;     // dO tiles: [3][BQ][D]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;
  const int ln = lane & 31;
  const int lh = lane >> 5;

  int bh, kt;
  bwd_work(p, p.n_ktiles, bh, kt);      // causal: low key tiles see the most queries
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int N = p.N;
  const long long tok = (long long)p.H * D;
  const long long head_base = ((long long)b * N * p.H + h) * D;
  const int k0 = kt * BK;
  const int kw0 = k0 + wave * 32;
  const int mykey = kw0 + ln;
  const int kr = mykey < N ? mykey : N - 1;

  const __bf16* __restrict__ qg = (const __bf16*)p.q + head_base;
  const __bf16* __restrict__ kg = (const __bf16*)p.k + head_base;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + head_base;
  const __bf16* __restrict__ gg = (const __bf16*)p.dout + head_base;

  // K^T and V^T fragments (B operands of S = Q K^T and dP = dO V^T): lane
  // (n = ln, h = lh) holds row mykey, columns 16 ks + 8 lh .. +7
  bf16x8 kf[NKS], vf[DK ? NKS : 1];
  {
    const u32x4* ks = (const u32x4*)(kg + (long long)kr * tok + 8 * lh);
    const u32x4* vs = (const u32x4*)(vg + (long long)kr * tok + 8 * lh);
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      kf[i] = __builtin_bit_cast(bf16x8, ks[2 * i]);
      if constexpr (DK) vf[i] = __builtin_bit_cast(bf16x8, vs[2 * i]);
    }
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      loaded(kf[i]);
      if constexpr (DK) loaded(vf[i]);
    }
  }
  const float c = p.c;

  const int n_q_all = (N + BQ - 1) / BQ;
  const int first = CAUSAL ? k0 / BQ : 0;
  const int nt = n_q_all > first ? n_q_all - first : 0;    // tiles of this work-group
  // the wave's keys see tile t (local index) unless all its queries precede them
  const int wfirst = CAUSAL ? max(kw0 / BQ - first, 0) : 0;
  const bool wave_on = kw0 < N;

  TileLoader<D, 4, BQ> ld;
  ld.init(wave & 3, lane, tok);
  const unsigned lds_q = (unsigned)(size_t)((ATTN_LDS __bf16*)qs_base);
  const unsigned lds_g = (unsigned)(size_t)((ATTN_LDS __bf16*)gs_base);
  const float* __restrict__ lse_h = p.lse + (long long)bh * N;
  const float* __restrict__ del_h = p.delta + (long long)bh * N;
  float row_lse = 0.f, row_del = 0.f;
  // tile u (local): Q, dO into buffer u % 3; its lse / D into registers of
  // wave 0 (lanes < BQ), written to LDS by store_rowv after the wait
  auto load_tile = [&](int u) {
    const int q0t = (first + u) * BQ;
    const unsigned nb = (unsigned)((u % 3) * TILE * 2);
    ld.load(qg, tok, lds_q + nb, q0t, N);
    ld.load(gg, tok, lds_g + nb, q0t, N);
    if (wave == 0 && lane < BQ) {
      const int r = min(q0t + lane, N - 1);
      row_lse = lse_h[r];
      row_del = del_h[r];
    }
  };
  auto store_rowv = [&](int u) {
    if (wave == 0 && lane < BQ) {
      rowv[u % 3][0][lane] = row_lse * kLog2e;
      rowv[u % 3][1][lane] = row_del;
    }
  };

  int qoff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qoff[ks] = ln * D + (((2 * ks + lh) ^ swz_b<D>(ln)) * 8);
  TrOffsets<D, NDB> tro;
  tro.init(lane);

  f32x16 dk[DK ? NDB : 1], dv[DV ? NDB : 1];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    if constexpr (DK) dk[db] = f32x16{};
    if constexpr (DV) dv[db] = f32x16{};
  }
  f32x16 s[NQB], dp[DK ? NQB : 1];
  bf16x8 pf[DV ? NQB : 1][2], dsf[DK ? NQB : 1][2];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    s[qb] = f32x16{};
    if constexpr (DK) dp[qb] = f32x16{};
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if constexpr (DV) pf[qb][g] = bf16x8{};
      if constexpr (DK) dsf[qb][g] = bf16x8{};
    }
  }

  // ---- X_u: the update of tile u, then S (and dP) of tile u+1
  auto phase_x = [&](auto up_tag, auto sd_tag, int u) {
    constexpr bool UP = decltype(up_tag)::value;
    constexpr bool SD = decltype(sd_tag)::value;
    __builtin_amdgcn_s_setprio(3);
    if constexpr (UP) {
      const __bf16* qt = qs_base + (u % 3) * TILE;
      const __bf16* gt = gs_base + (u % 3) * TILE;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int rowb = (32 * qb + 16 * g) * D;
            if constexpr (DV) {
              const bf16x8 ga = tr_operand(gt + rowb, tro.lo[db], tro.hi[db]);
              dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, pf[qb][g], dv[db], 0, 0, 0);
            }
            if constexpr (DK) {
              const bf16x8 qa = tr_operand(qt + rowb, tro.lo[db], tro.hi[db]);
              dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dsf[qb][g], dk[db], 0, 0, 0);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SD) {
      const __bf16* qt = qs_base + ((u + 1) % 3) * TILE;
      const __bf16* gt = gs_base + ((u + 1) % 3) * TILE;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const bf16x8 qa = *(const bf16x8*)(qt + qb * 32 * D + qoff[ks]);
          s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], ks == 0 ? f32x16{} : s[qb], 0, 0, 0);
          if constexpr (DK) {
            const bf16x8 ga = *(const bf16x8*)(gt + qb * 32 * D + qoff[ks]);
            dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[ks], ks == 0 ? f32x16{} : dp[qb], 0, 0, 0);
          }
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- Y_u: P (and dS) of tile u+1 (queries q0t ..), packed to bf16
  auto phase_y = [&](auto masked_tag, int u) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int buf = (u + 1) % 3;
    const int q0t = (first + u + 1) * BQ;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // register r holds query q0t + 32 qb + 8 (r/4) + 4 lh + r%4 of key mykey
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        u32x4 wp, wd;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int rb = 8 * g + 4 * half;                        // registers rb .. rb+3
          const int qi = 32 * qb + 8 * (rb >> 2) + 4 * lh;        // their first tile row
          const f32x4 lv = *(const f32x4*)&rowv[buf][0][qi];
          float pv[4], dsv[4];
          f32x4 dv4;
          if constexpr (DK) dv4 = *(const f32x4*)&rowv[buf][1][qi];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            float pe = fast_exp2(__builtin_fmaf(s[qb][rb + x], c, -lv[x]));
            if constexpr (MASKED) {
              const int q = q0t + qi + x;
              if (q >= N || (CAUSAL && mykey > q)) pe = 0.f;
            }
            pv[x] = pe;
            if constexpr (DK) dsv[x] = pe * (dp[qb][rb + x] - dv4[x]);
          }
          if constexpr (DV) {
            wp[2 * half] = pack_bf16x2(pv[0], pv[1]);
            wp[2 * half + 1] = pack_bf16x2(pv[2], pv[3]);
          }
          if constexpr (DK) {
            wd[2 * half] = pack_bf16x2(dsv[0], dsv[1]);
            wd[2 * half + 1] = pack_bf16x2(dsv[2], dsv[3]);
          }
        }
        if constexpr (DV) pf[qb][g] = __builtin_bit_cast(bf16x8, wp);
        if constexpr (DK) dsf[qb][g] = __builtin_bit_cast(bf16x8, wd);
      }
    }
  };

  if (grp == 0 && nt > 0) load_tile(0);
  wait_vmem();
  if (nt > 0) store_rowv(0);
  __syncthreads();

  using T_ = std::true_type;
  using F_ = std::false_type;
  const int n_phases = 2 * nt + 2;
  for (int ph = 0; ph < n_phases; ++ph) {
    if (grp == 0 && (ph & 1) == 0) {
      const int u = ph >> 1;
      if (u + 1 < nt) load_tile(u + 1);
    }
    const int q = ph - grp;
    if (q >= 0 && wave_on) {
      if ((q & 1) == 0) {
        const int u = (q >> 1) - 1;
        const bool up = u >= wfirst && u < nt;
        const bool sd = u + 1 >= wfirst && u + 1 < nt;
        if (up && sd)
          phase_x(T_{}, T_{}, u);
        else if (sd)
          phase_x(F_{}, T_{}, u);
        else if (up)
          phase_x(T_{}, F_{}, u);
      } else {
        const int u = (q - 3) / 2;
        if (u + 1 >= wfirst && u + 1 < nt) {
          const int q0t = (first + u + 1) * BQ;
          if ((q0t + BQ > N) || (CAUSAL && q0t < kw0 + 31))
            phase_y(T_{}, u);
          else
            phase_y(F_{}, u);
        }
      }
    }
    if (grp == 0 && (ph & 1) == 1) {
      wait_vmem();
      const int u = ph >> 1;
      if (u + 1 < nt) store_rowv(u + 1);
    }
    __syncthreads();
  }

  if (mykey < N) {
    if constexpr (DK) store_rows<NDB>((__bf16*)p.dk + head_base + (long long)mykey * tok, dk, p.scale, lh);
    if constexpr (DV) store_rows<NDB>((__bf16*)p.dv + head_base + (long long)mykey * tok, dv, 1.f, lh);
  }
}

// ---------------------------------------------------------------------------
// dK and dV together, one wave per SIMD: per (batch, head, 128 key rows).
// Each of the 4 waves owns 32 keys: their K and V rows stay in registers
// (the B operands of S and dP) and dK^T, dV^T (32 keys x D fp32) accumulate
// in the accumulation registers, which a wave has to itself when it is
// alone on its SIMD.  64-query Q / dO tiles stream through three LDS
// buffers (with their lse and D values); the wave walks them in 32-query
// blocks t and overlaps, within its own instruction stream, the vector work
// of one block with the matrix-core work of the next:
//   iteration t:  S_{t+1} = Q_{t+1} K^T, dP_{t+1} = dO_{t+1} V^T
//                 (matrix cores) together with P_t, dS_t (vector ALU), then
//                 dV^T += dO_t^T P_t, dK^T += Q_t^T dS_t.
// Five products per (query, key) pair of the backward pass are here (S, dP,
// dV, dK) or in the dQ kernel (S, dP again, dQ).  Tile j+1 is loaded two
// iterations before its first use; one barrier per tile, after block 2j,
// publishes it and frees the buffer of tile j-1 for tile j+2.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_1w_kernel(BwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int NW = 4;
  constexpr int BK = NW * 32, BQ = 64, NBUF = 3;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int TILE = BQ * D;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * NBUF * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 vsm[BK * D];        // the work-group's V rows
  __shared__ __attribute__((aligned(16))) float rowv[NBUF][2][BQ];   // [buffer][lse2, D][query]
  __bf16* qs_base = smem;                   // Q tiles:  [NBUF][BQ][D]
  __bf16* gs_base = smem + NBUF * TILE;     // dO tiles: [NBUF][BQ][D]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
  const int ln = lane & 31;
  const int lh = lane >> 5;

  int bh, kt;
  bwd_work(p, p.n_ktiles, bh, kt);      // causal: low key tiles see the most queries
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int N = p.N;
  const long long tok = (long long)p.H * D;
  const long long head_base = ((long long)b * N * p.H + h) * D;
  const int k0 = kt * BK;
  const int kw0 = k0 + wave * 32;
  const int mykey = kw0 + ln;
  const int kr = mykey < N ? mykey : N - 1;

  const __bf16* __restrict__ qg = (const __bf16*)p.q + head_base;
  const __bf16* __restrict__ kg = (const __bf16*)p.k + head_base;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + head_base;
  const __bf16* __restrict__ gg = (const __bf16*)p.dout + head_base;

  // K^T fragments (B operand of S = Q K^T): lane (n = ln, h = lh) holds row
  // mykey, columns 16 ks + 8 lh .. +7.  The V^T fragments (B operand of
  // dP = dO V^T) are read from the work-group's V rows in LDS.
  bf16x8 kf[NKS];
  {
    const u32x4* ks = (const u32x4*)(kg + (long long)kr * tok + 8 * lh);
#pragma unroll
    for (int i = 0; i < NKS; ++i) kf[i] = __builtin_bit_cast(bf16x8, ks[2 * i]);
  }
  const float c = p.c;

  const int n_q_all = (N + BQ - 1) / BQ;
  const int first = CAUSAL ? k0 / BQ : 0;
  const int nt = n_q_all - first;           // >= 1: k0 < N
  const int nblk = 2 * nt;

  TileLoader<D, NW, BQ> ld;
  ld.init(wave, lane, tok);
  const unsigned lds_q = (unsigned)(size_t)((ATTN_LDS __bf16*)qs_base);
  const unsigned lds_g = (unsigned)(size_t)((ATTN_LDS __bf16*)gs_base);
  const float* __restrict__ lse_h = p.lse + (long long)bh * N;
  const float* __restrict__ del_h = p.delta + (long long)bh * N;
  float row_lse = 0.f, row_del = 0.f;
  // tile j (local): Q, dO into buffer j % 3; its lse / D into registers of
  // wave 0, written to LDS by store_rowv after the wait
  auto load_tile = [&](int j) {
    j = __builtin_amdgcn_readfirstlane(j);
    const int q0t = (first + j) * BQ;
    const unsigned nb = (unsigned)((j % NBUF) * TILE * 2);
    ld.load(qg, tok, lds_q + nb, q0t, N);
    ld.load(gg, tok, lds_g + nb, q0t, N);
    if (wave == 0) {
      const int r = min(q0t + lane, N - 1);
      row_lse = lse_h[r];
      row_del = del_h[r];
    }
  };
  auto store_rowv = [&](int j) {
    if (wave == 0) {
      rowv[j % NBUF][0][lane] = row_lse * kLog2e;
      rowv[j % NBUF][1][lane] = row_del;
    }
  };

  int qoff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qoff[ks] = ln * D + (((2 * ks + lh) ^ swz_b<D>(ln)) * 8);
  TrOffsets<D, NDB> tro;
  tro.init(lane);
  const __bf16* vw = vsm + wave * 32 * D;   // the wave's 32 V rows

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  // S and dP of blocks t and t+1 (slot = block & 1); P and dS of blocks t
  // and t-1 (the B operands of the update), same slots
  f32x16 s[2], dp[2];
  bf16x8 pf[2][2], dsf[2][2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      pf[sl][g] = bf16x8{};
      dsf[sl][g] = bf16x8{};
    }
  constexpr int NU = 4 * NDB;             // update products: (g, db, dV | dK)
  constexpr int UA = 4;                   // update operands read ahead
  bf16x8 ua[NU];                          // update operands (transposed rows)
  // update product u: g = u / (2 NDB), db = (u / 2) % NDB, dV (u even) or dK
  // (u odd); its A operand is dO^T or Q^T of the block's rows 16 g .. +15
  auto u_read = [&](int u, const __bf16* qb, const __bf16* gb) __attribute__((always_inline)) {
    const int g = u / (2 * NDB), db = (u >> 1) % NDB;
    ua[u] = tr_operand(((u & 1) ? qb : gb) + 16 * g * D, tro.lo[db], tro.hi[db]);
  };
  auto u_mfma = [&](int u, int sl) __attribute__((always_inline)) {
    const int g = u / (2 * NDB), db = (u >> 1) % NDB;
    if (u & 1)
      dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[u], dsf[sl][g], dk[db], 0, 0, 0);
    else
      dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[u], pf[sl][g], dv[db], 0, 0, 0);
  };

  // S, dP of block 0 (buffer 0, rows 0-31) into slot 0
  auto sd0 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 qa = *(const bf16x8*)(qs_base + qoff[ks]);
      const bf16x8 ga = *(const bf16x8*)(gs_base + qoff[ks]);
      const bf16x8 vb = *(const bf16x8*)(vw + qoff[ks]);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], ks == 0 ? f32x16{} : s[0], 0, 0, 0);
      dp[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vb, ks == 0 ? f32x16{} : dp[0], 0, 0, 0);
    }
  };

  // Iteration t = 2 j + SL of tile j (block t = rows 32 SL .. 32 SL + 31 of
  // the tile): the update of block t-1, S and dP of block t+1, and P and dS
  // of block t.  It is written as 2 NU regions of one matrix-core product
  // each, in a fixed order (scheduling fences between regions):
  //   regions 0 .. NU-1:     update products of block t-1 (P, dS of slot SN);
  //   regions NU .. 2NU-1:   S, dP of block t+1, k-step by k-step (slot SN);
  // with the vector work of block t (slot SL) spread over all of them: its
  // 16 (query, key) values per lane go in 8 pairs, pair p taking regions
  // 4p+1 (exponential), 4p+2 (dS) and 4p+3 (packing to bf16).  LDS operands
  // are read ahead: update operands UA products ahead (the first UA in the
  // previous iteration's last regions), S / dP operands two k-steps ahead,
  // a quarter's lse and D values four regions ahead.  The buffer offsets pass
  // through an empty asm so that each iteration forms its own LDS addresses
  // (one per lane pattern; the dO tile and row offsets are immediates).
  // Block -1 (before the first) is an update with P = dS = 0 on block 0's
  // rows; after the last block the S, dP products read a stale buffer and
  // are discarded.
  auto iter = [&](auto masked_tag, auto slot_tag, int j) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int SL = decltype(slot_tag)::value;
    constexpr int SN = SL ^ 1;
    constexpr int NR = 2 * NU;
    constexpr int qb0 = 32 * SL;
    const int q0 = (first + j) * BQ + qb0;
    const int buf = j % NBUF;
    int ecur = buf * TILE + qb0 * D;                                   // block t
    int enxt = SL ? ((j + 1) % NBUF) * TILE : ecur + 32 * D;           // block t+1
    int eprv = SL ? buf * TILE : (j > 0 ? ((j + NBUF - 1) % NBUF) * TILE + 32 * D : ecur);
    asm volatile("" : "+s"(ecur), "+s"(enxt), "+s"(eprv));
    const __bf16* qc = qs_base + ecur;
    const __bf16* gc = gs_base + ecur;
    const __bf16* qn = qs_base + enxt;
    const __bf16* gn = gs_base + enxt;
    const __bf16* qp = qs_base + eprv;
    const __bf16* gp = gs_base + eprv;

    bf16x8 qa[NKS], ga[NKS], vb[NKS];
    f32x4 lv[4], dv4[4];
    float pe[16], dsv[16];
    auto rows = [&](int x) __attribute__((always_inline)) {
      lv[x] = *(const f32x4*)&rowv[buf][0][qb0 + 8 * x + 4 * lh];
      dv4[x] = *(const f32x4*)&rowv[buf][1][qb0 + 8 * x + 4 * lh];
    };
    // pair p = values 2p, 2p+1 (registers of quarter x = p / 2)
    auto stage_exp = [&](int p) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 2 * p + i, x = r >> 2, e = r & 3;
        float v = fast_exp2(__builtin_fmaf(s[SL][r], c, -lv[x][e]));
        if constexpr (MASKED) {
          const int q = q0 + 8 * x + 4 * lh + e;
          if (q >= N || (CAUSAL && mykey > q)) v = 0.f;
        }
        pe[r] = v;
      }
    };
    auto stage_ds = [&](int p) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 2 * p + i, x = r >> 2, e = r & 3;
        dsv[r] = pe[r] * (dp[SL][r] - dv4[x][e]);
      }
    };
    auto stage_pack = [&](int p) __attribute__((always_inline)) {
      const int g = p >> 2, w = p & 3;
      u32x4 wp = __builtin_bit_cast(u32x4, pf[SL][g]);
      u32x4 wd = __builtin_bit_cast(u32x4, dsf[SL][g]);
      wp[w] = pack_bf16x2(pe[2 * p], pe[2 * p + 1]);
      wd[w] = pack_bf16x2(dsv[2 * p], dsv[2 * p + 1]);
      // computed here, not where first used (after the tile's barrier)
      asm volatile("" : "+v"(wp), "+v"(wd));
      pf[SL][g] = __builtin_bit_cast(bf16x8, wp);
      dsf[SL][g] = __builtin_bit_cast(bf16x8, wd);
    };

    rows(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      // reads ahead
      if (r + UA < NU) u_read(r + UA, qp, gp);
      if (r >= NU - 4 && r < NR - 4 && (r & 1) == 0) {
        const int ks = (r - (NU - 4)) / 2;
        qa[ks] = *(const bf16x8*)(qn + qoff[ks]);
        ga[ks] = *(const bf16x8*)(gn + qoff[ks]);
        vb[ks] = *(const bf16x8*)(vw + qoff[ks]);
      }
      if (r >= NR - UA) u_read(r - (NR - UA), qc, gc);   // the next iteration's first
      if ((r & 7) == 5 && (r >> 3) < 3) rows((r >> 3) + 1);
      // the region's product
      if (r < NU) {
        u_mfma(r, SN);
      } else {
        const int ks = (r - NU) >> 1;
        if ((r & 1) == 0)
          s[SN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], kf[ks], ks == 0 ? f32x16{} : s[SN], 0, 0, 0);
        else
          dp[SN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[ks], vb[ks], ks == 0 ? f32x16{} : dp[SN], 0, 0, 0);
      }
      // the vector work of block t
      if ((r & 3) == 1) stage_exp(r >> 2);
      if ((r & 3) == 2) stage_ds(r >> 2);
      if ((r & 3) == 3) stage_pack(r >> 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the update of the last block (a tile's second: slot 1), after the loop
  auto last_update = [&](int t) __attribute__((always_inline)) {
    int ecur = ((t >> 1) % NBUF) * TILE + 32 * D;
    asm volatile("" : "+s"(ecur));
    const __bf16* qc = qs_base + ecur;
    const __bf16* gc = gs_base + ecur;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (u + UA < NU) u_read(u + UA, qc, gc);
      u_mfma(u, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // the P / dS of tile j need the mask: causal diagonal (or keys after all
  // its queries) or rows past N
  auto tile_masked = [&](int j) {
    const int q0 = (first + j) * BQ;
    return (q0 + BQ > N) || (CAUSAL && q0 < kw0 + 31);
  };
  // tile j: its two blocks, with the barrier between them that publishes
  // tile j+1 and frees the buffer of tile j-1 for tile j+2
  auto tile = [&](auto masked_tag, int j) __attribute__((always_inline)) {
    iter(masked_tag, std::integral_constant<int, 0>{}, j);
    wait_vmem();                  // tile j+1 (loaded two iterations ago)
    if (j + 1 < nt) store_rowv(j + 1);
    __syncthreads();
    if (j + 2 < nt) load_tile(j + 2);
    iter(masked_tag, std::integral_constant<int, 1>{}, j);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  {
    TileLoader<D, NW, BK> ldv;
    ldv.init(wave, lane, tok);
    ldv.load(vg, tok, (unsigned)(size_t)((ATTN_LDS __bf16*)vsm), k0, N);
  }
  load_tile(0);
  wait_vmem();
  store_rowv(0);
  __syncthreads();
  if (nt > 1) load_tile(1);
  sd0();
#pragma unroll
  for (int u = 0; u < UA; ++u) u_read(u, qs_base, gs_base);   // block -1: block 0's rows
  // masked tiles are a prefix (causal) and possibly the last one
  int j = 0;
  for (; j + 1 < nt && tile_masked(j); ++j) tile(T_{}, j);
  for (; j + 1 < nt; ++j) tile(F_{}, j);
  if (tile_masked(nt - 1))
    tile(T_{}, nt - 1);
  else
    tile(F_{}, nt - 1);
  last_update(nblk - 1);

  if (mykey < N) {
    store_rows<NDB>((__bf16*)p.dk + head_base + (long long)mykey * tok, dk, p.scale, lh);
    store_rows<NDB>((__bf16*)p.dv + head_base + (long long)mykey * tok, dv, 1.f, lh);
  }
}

// ---------------------------------------------------------------------------
// host-side launch (called by the C ABI in attn_api.cpp)
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(BwdParams prm, hipStream_t stream) {
  const long long rows = (long long)prm.B * prm.N * prm.H;
  const int grid_delta = (int)((rows + 15) / 16);
  hipError_t e = launch_kernel(attn_bwd_delta_kernel<D>, dim3(grid_delta), dim3(256), stream, prm);
  if (e != hipSuccess) return e;
  const int grid = prm.B * prm.H * prm.n_tiles;
  e = launch_kernel(attn_bwd_dq_kernel<D, CAUSAL>, dim3(grid), dim3(512), stream, prm);
  if (e != hipSuccess) return e;
  if constexpr (D == 128) {
    prm.n_ktiles = (prm.N + 127) / 128;
    return launch_kernel(attn_bwd_dkdv_1w_kernel<D, CAUSAL>, dim3(prm.B * prm.H * prm.n_ktiles),
                         dim3(256), stream, prm);
  } else {
    prm.n_ktiles = prm.n_tiles;
    return launch_kernel(attn_bwd_dkdv_kernel<D, CAUSAL, 3>, dim3(grid), dim3(512), stream, prm);
  }
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* delta, int B, int H, int N, int d, int causal, float scale,
                           hipStream_t stream) {
  BwdParams prm = {};
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = o;
  prm.lse = lse;
  prm.dout = dout;
  prm.dq = dq;
  prm.dk = dk;
  prm.dv = dv;
  prm.delta = delta;
  prm.B = B;
  prm.H = H;
  prm.N = N;
  prm.n_tiles = (N + 255) / 256;
  prm.tile_major = causal && prm.n_tiles < 32 && (B * H) % 8 == 0;
  prm.scale = scale;
  prm.c = scale * kLog2e;
  if (d == 128) return causal ? launch_bwd_t<128, true>(prm, stream) : launch_bwd_t<128, false>(prm, stream);
  return causal ? launch_bwd_t<64, true>(prm, stream) : launch_bwd_t<64, false>(prm, stream);
}

}  // namespace attn
