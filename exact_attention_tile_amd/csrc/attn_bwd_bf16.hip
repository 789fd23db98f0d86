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
// Three kernels, enqueued in order on the caller's stream:
//   delta : D_i for every row (a dot product of two rows), into the caller's
//           fp32 workspace [B][H][N];
//   dQ    : one work-group per (batch, head, 256 queries); each wave owns 32
//           query columns and streams 64-key K/V tiles through LDS:
//             S^T = K Q^T, dP^T = V dO^T (A = K / V rows, B = Q^T / dO^T in
//             VGPRs), dS^T = P^T (dP^T - D), dQ^T += K^T dS^T (A = K^T from
//             transposing LDS reads, B = dS^T packed to bf16);
//   dK/dV : key-owned waves (lane = key) streaming 64-query Q / dO tiles
//           (plus their lse and D values) through LDS:
//             S = Q K^T, dP = dO V^T (A = Q / dO rows), dS = P (dP - D),
//             dV^T += dO^T P, dK^T += Q^T dS (A = dO^T / Q^T from transposing
//             LDS reads, B = P / dS packed to bf16).
//           At d = 64 each of the 8 waves of a 256-key work-group does all
//           of it for its 32 keys; at d = 128 the two waves of a SIMD share
//           32 keys, one computing S, P and dV, the other dP, dS and dK
//           (P passed through LDS).  S and dP are computed once per (query,
//           key) pair here and once more in the dQ kernel: 7 products per
//           pair where the chain rule has 5.
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
  int items;         // work items of the kernel launched: (batch*head, tile) pairs
  int persist;       // 1: gridDim.x work-groups (a multiple of 8) loop over the items
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
// 1 KiB pieces of a [ROWS][D] bf16 tile with global_load_lds_dwordx4
// (lds_dma_*: lane l fills bytes [16 l, 16 l + 16) of a piece), choosing
// each lane's source chunk so that the tile lands swizzled; rows past N are
// clamped to row N-1.  The loads share M0 in groups of four, so the offset
// of piece i is stored less 1024 (i % 4) (still >= 0: piece i starts at
// least that many bytes into the tile).
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
      go[i] = (unsigned)(((long long)r * tok + (pc ^ swz_b<D>(r)) * 8) * 2) - (unsigned)((i & 3) * 1024);
    }
    lds_wave = __builtin_amdgcn_readfirstlane((unsigned)(wave * LPW * 1024));
  }
  // rows row0 .. row0+ROWS-1 of the tensor at src (element (row, 0) = src + row*tok)
  // The byte offset of row0 is one 32x32 -> 64-bit product: the loads are
  // issued in vector phases, where a lone wave issues every instruction
  // slowly, scalar ones included.
  __device__ void load(const __bf16* src, long long tok, unsigned lds_buf, int row0, int N) const {
    const unsigned la0 = lds_buf + lds_wave;
    const __bf16* base =
        (const __bf16*)((const char*)src + (unsigned long long)(unsigned)row0 * (unsigned)(tok * 2));
    if (__builtin_expect(row0 + ROWS <= N, 1)) {
      lds_dma_tile_s<LPW>(la0, go, base);
    } else {
      const void* g[LPW];
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const long long back = (long long)(row0 + row[i] < N ? 0 : row0 + row[i] - (N - 1)) * tok;
        g[i] = base + (long long)(go[i] / 2) - back;
      }
      lds_dma_tile_v<LPW>(la0, g);
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
__device__ __forceinline__ int xcd_order(int L, int total) {
  if ((total & 7) != 0) return L;
  return (L & 7) * (total >> 3) + (L >> 3);
}

// (batch*head, rank) of work-group L for n tiles per head; rank 0 is the
// head's longest tile.  Head-major within each XCD (xcd_order), except for
// causal calls with few tiles per head (tile_major, B*H divisible by 8):
// their causal tile lengths do not pair up over an XCD's 32 CUs, so each XCD
// keeps its share of the heads but runs the longest tile of every head
// first, then the next longest.
__device__ __forceinline__ void bwd_work(const BwdParams& p, int n, int L, int& bh, int& rank) {
  if (p.tile_major) {
    const int hx = (p.B * p.H) >> 3;
    const int k = L >> 3;
    rank = k / hx;
    bh = (L & 7) * hx + (k - rank * hx);
    return;
  }
  const int Lx = xcd_order(L, p.items);
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
template <int D, bool CAUSAL, bool LOOP>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_kernel(BwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int BR = 256, BC = 64;
  constexpr int NKB = BC / 32, NKK = BC / 16, NKS = D / 16, NDB = D / 32;
  constexpr int TILE = BC * D;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * TILE];
  __bf16* ks_base = smem;
  __bf16* vs_base = smem + 2 * TILE;

  // one work item per step.  LOOP (persistent launches, item_of_n): an
  // item's first loads go into LDS only after every wave has passed the
  // previous item's last barrier, and the lane's values are derived anew in
  // every item (taken out of the loop they would stay live through it and
  // cost registers).  Without LOOP the body is compiled straight, once.
  constexpr int kMaxSteps = LOOP ? 0x7fffffff : 1;
  for (int step = 0; step < kMaxSteps; ++step) {
  int L;
  if (!item_of_n(p.items, p.persist, step, L)) break;
  int tid = threadIdx.x;
  if constexpr (LOOP) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31;
  const int lh = lane >> 5;
  int bh, rank;
  bwd_work(p, p.n_tiles, L, bh, rank);
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
  }   // work items
}

// ---------------------------------------------------------------------------
// dK and dV at D = 64: per (batch, head, 256 key rows); 64-query Q / dO
// tiles.  Each of the 8 waves (two per SIMD) owns 32 keys and keeps their K
// and V rows and both 32 x 64 fp32 accumulators in registers (at D = 128
// these do not fit the 256 registers of a wave that shares its SIMD:
// attn_bwd_dkdv_pair_kernel below splits the work between two waves).
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool LOOP>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  static_assert(D == 64, "head dim 64 (128: attn_bwd_dkdv_pair_kernel)");
  constexpr bool DV = true;
  constexpr bool DK = true;
  constexpr int NW = 8;
  constexpr int BK = NW * 32, BQ = 64;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int TILE = BQ * D;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * TILE];
  __shared__ __attribute__((aligned(16))) float rowv[2][2][BQ];   // [buffer][lse2, D][query]
  __bf16* qs_base = smem;
  __bf16* gs_base = smem + 2 * TILE;

  // one work item per step.  LOOP (persistent launches, item_of_n): an
  // item's first loads go into LDS only after every wave has passed the
  // previous item's last barrier, and the lane's values are derived anew in
  // every item (taken out of the loop they would stay live through it and
  // cost registers).  Without LOOP the body is compiled straight, once.
  constexpr int kMaxSteps = LOOP ? 0x7fffffff : 1;
  for (int step = 0; step < kMaxSteps; ++step) {
  int L;
  if (!item_of_n(p.items, p.persist, step, L)) break;
  int tid = threadIdx.x;
  if constexpr (LOOP) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31;
  const int lh = lane >> 5;
  int bh, kt;
  bwd_work(p, p.n_ktiles, L, bh, kt);   // causal: low key tiles see the most queries
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
  }   // work items
}

// ---------------------------------------------------------------------------
// dK and dV with each key block's work split between the two waves of a
// SIMD, per (batch, head, 128 key rows), streaming 64-query Q / dO tiles.
// Wave w < 4 (the P wave) and wave w + 4 (the dS wave) own the same 32 keys
// k0 + 32 w .. +31.  The P wave keeps their K rows (B operand) and dV^T:
//   S = Q K^T,  P = exp2(S scale log2(e) - lse log2(e)),  dV^T += dO^T P,
// and hands P (fp32) to the dS wave through LDS; the dS wave keeps their V
// rows and dK^T:
//   dP = dO V^T,  dS = P (dP - D),  dK^T += Q^T dS.
// The two alternate, one phase apart (a barrier ends every phase):
//   phase 2i+2:  P wave  dV(i), S(i+1)   (matrix cores)  | dS wave  dS(i)
//   phase 2i+3:  P wave  P(i+1)          (vector ALU)    | dS wave  dK(i), dP(i+1)
// (phase 0: S(0) | dP(0); phase 1: P(0) | -), so one wave of a SIMD issues
// products while the other issues its vector work.  S and dP are computed
// once per (query, key) pair.  Q tile i is read in phases 2i .. 2i+3 and dO
// tile i in phases 2i+1 and 2i+2, so Q tiles rotate through three LDS
// buffers and dO tiles through two.  Each wave issues its share of the next
// tile's loads at the start of its vector phase, where they delay neither
// wave's products: the dS waves load Q and lse (tile k+1 in phase 2k), the
// P waves dO and D (tile k+1 in phase 2k+1); each waits for its own loads
// at the end of the following phase.  The accumulation order per key is the
// tiles', then 16-query groups, so the results do not depend on the split.
// A matrix-core phase is one stream of 32 products whose operands are read
// from LDS four products ahead, the first four at the end of the vector
// phase before it; the swizzled offsets of k-step ks and column block db are
// the first ones XOR 16 ks and XOR 32 db (elements).
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool LOOP>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_pair_kernel(BwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int KW = 4;                   // key groups of 32 (one per SIMD)
  constexpr int BK = KW * 32, BQ = 64, NB = 3;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int TILE = BQ * D;
  constexpr int PF = 4;                   // LDS operands read this many products ahead
  __shared__ __attribute__((aligned(16))) __bf16 qsm[NB * TILE];       // Q tiles, 3 buffers
  __shared__ __attribute__((aligned(16))) __bf16 gsm[2 * TILE];        // dO tiles, 2 buffers
  __shared__ __attribute__((aligned(16))) __bf16 vsm[BK * D];          // the work-group's V rows
  __shared__ __attribute__((aligned(16))) f32x4 pbuf[KW][8][64];   // [key group][(qb, quarter)][lane]
  __shared__ __attribute__((aligned(16))) float rowv[NB][2][BQ];   // [buffer][lse2, D][query]

  // one work item per step.  LOOP (persistent launches, item_of_n): an
  // item's first loads go into LDS only after every wave has passed the
  // previous item's last barrier, and the lane's values are derived anew in
  // every item (taken out of the loop they would stay live through it and
  // cost registers).  Without LOOP the body is compiled straight, once.
  constexpr int kMaxSteps = LOOP ? 0x7fffffff : 1;
  for (int step = 0; step < kMaxSteps; ++step) {
  int L;
  if (!item_of_n(p.items, p.persist, step, L)) break;
  int tid = threadIdx.x;
  if constexpr (LOOP) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
  const int role = wave >> 2;                                  // 0: P wave, 1: dS wave
  const int kgrp = wave & 3;
  const int ln = lane & 31;
  const int lh = lane >> 5;
  int bh, kt;
  bwd_work(p, p.n_ktiles, L, bh, kt);   // causal: low key tiles see the most queries
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int N = p.N;
  const long long tok = (long long)p.H * D;
  const long long head_base = ((long long)b * N * p.H + h) * D;
  const int k0 = kt * BK;
  const int kw0 = k0 + kgrp * 32;
  const int mykey = kw0 + ln;
  const int kr = mykey < N ? mykey : N - 1;
  const float c = p.c;

  const int n_q_all = (N + BQ - 1) / BQ;
  const int first = CAUSAL ? k0 / BQ : 0;
  const int nt = n_q_all - first;                          // >= 1: k0 < N
  const int n_phases = 2 * nt + 2;

  // this wave's share of the tile loads, issued in its vector phases (the
  // matrix-core phase of its partner wave, which they would otherwise
  // delay): Q and lse (dS waves, lr = 0; tile k+1 at the start of phase 2k,
  // waited for at the end of phase 2k+1) or dO and D (P waves, lr = 1; tile
  // k+1 at the start of phase 2k+1, waited for at the end of phase 2k+2).
  // Q tile i is read in phases 2i .. 2i+3, dO tile i in phases 2i+1 and
  // 2i+2, hence three Q buffers and two dO buffers.
  const int lr = 1 - role;
  const __bf16* __restrict__ src = (const __bf16*)(lr ? p.dout : p.q) + head_base;
  const float* __restrict__ rsrc = (lr ? p.delta : p.lse) + (long long)bh * N;
  TileLoader<D, KW, BQ> ld;
  ld.init(kgrp, lane, tok);
  const unsigned lds_dst = (unsigned)(size_t)((ATTN_LDS __bf16*)(lr ? gsm : qsm));
  float row_val = 0.f;
  auto load_tile = [&](int u) {
    const int q0t = (first + u) * BQ;
    // the buffer: u mod 2 (dO) or u mod NB (Q), each with a constant
    // divisor (a run-time one costs a full integer division, VALU
    // reciprocal included, in the loading wave's vector phase)
    const int slot = lr ? (u & 1) : (u % NB);
    ld.load(src, tok, lds_dst + (unsigned)(slot * TILE * 2), q0t, N);
    if (kgrp == 0) row_val = rsrc[min(q0t + lane, N - 1)];
  };
  auto store_rowv = [&](int u) {
    if (kgrp == 0) rowv[u % NB][lr][lane] = lr ? row_val : row_val * kLog2e;
  };
  // the tile loads and barriers every wave takes part in, around phase ph
  auto phase_begin = [&](int ph) {
    const int k = (ph - lr) >> 1;
    if (((ph - lr) & 1) == 0 && ph >= lr && k + 1 < nt) load_tile(k + 1);
  };
  auto phase_end = [&](int ph) {
    const int k = (ph - 1 - lr) >> 1;
    if (((ph - 1 - lr) & 1) == 0 && ph >= 1 + lr) {
      wait_vmem();
      if (k + 1 < nt) store_rowv(k + 1);
    }
    __syncthreads();
  };
  // the end of a vector phase that read the next phase's first PF operands
  // (2 PF LDS reads, issued last): the barrier waits for this wave's earlier
  // LDS accesses, whose writes the other waves read next, but not for those
  // reads (LDS accesses complete in order).  No tile load is awaited at the
  // end of a vector phase; the general form is kept for that case.
  auto phase_end_pre = [&](int ph) {
    const int k = (ph - 1 - lr) >> 1;
    if (((ph - 1 - lr) & 1) == 0 && ph >= 1 + lr) {
      wait_vmem();
      if (k + 1 < nt) store_rowv(k + 1);
      __syncthreads();
    } else {
      asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(2 * PF) : "memory");
    }
  };

  // element offsets: row reads (k-step 0) and transposing reads (column
  // block 0); the others are these XOR 16 ks / XOR 32 db
  const int qoff0 = ln * D + ((lh ^ swz_b<D>(ln)) * 8);
  TrOffsets<D, 1> tro;
  tro.init(lane);

  // the B operand rows of this wave's keys: K in registers (P wave); V from
  // the work-group's V rows in LDS (dS wave)
  bf16x8 bf[NKS];
  if (role == 0) {
    const u32x4* rs = (const u32x4*)((const __bf16*)p.k + head_base + (long long)kr * tok + 8 * lh);
#pragma unroll
    for (int i = 0; i < NKS; ++i) bf[i] = __builtin_bit_cast(bf16x8, rs[2 * i]);
  } else {
    TileLoader<D, KW, BK> ldv;
    ldv.init(kgrp, lane, tok);
    ldv.load((const __bf16*)p.v + head_base, tok, (unsigned)(size_t)((ATTN_LDS __bf16*)vsm), k0, N);
  }

  load_tile(0);
  wait_vmem();
  store_rowv(0);
  if (role == 0) {
#pragma unroll
    for (int i = 0; i < NKS; ++i) loaded(bf[i]);
  }
  __syncthreads();

  f32x16 acc2[2];                         // S (P wave) or dP (dS wave) of a tile
  f32x16 acc[NDB];                        // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  bf16x8 pk[2][2];                        // [qb][g]: P or dS, packed
  // One matrix-core phase as one stream of products, whose LDS operands are
  // read PF products ahead across the join of its two parts:
  //   the update of tile uu: dV^T += dO^T P (P wave) or dK^T += Q^T dS (dS
  //   wave); A = the tile's dO or Q rows, transposed; B = the packed P or dS;
  //   the scores of tile us: S = Q K^T (P wave) or dP = dO V^T (dS wave), 2
  //   blocks of 32 queries; A = the tile's Q or dO rows, B = this wave's K
  //   or V rows.
  // The first phase has no update and the last no scores.  With PRE the
  // first PF operands were read at the end of the vector phase before
  // (pre_read), so the first product does not wait for LDS after the barrier.
  bf16x8 apre[PF];
  auto upd_operand = [&](const __bf16* tu, int lo, int hi, int i) __attribute__((always_inline)) {
    const int qb = i / (2 * NDB), g = (i / NDB) & 1, db = i % NDB;
    return tr_operand(tu + (32 * qb + 16 * g) * D, lo ^ (32 * db), hi ^ (32 * db));
  };
  auto upd_tile = [&](auto role_tag, int uu, int& lo, int& hi) __attribute__((always_inline)) {
    constexpr int R = decltype(role_tag)::value;
    int eb = (uu % (R ? NB : 2)) * TILE;
    lo = tro.lo[0];
    hi = tro.hi[0];
    asm volatile("" : "+s"(eb), "+v"(lo), "+v"(hi));
    return (R ? qsm : gsm) + eb;
  };
  auto pre_read = [&](auto role_tag, int uu) __attribute__((always_inline)) {
    int lo, hi;
    const __bf16* tu = upd_tile(role_tag, uu, lo, hi);
#pragma unroll
    for (int i = 0; i < PF; ++i) apre[i] = upd_operand(tu, lo, hi, i);
  };
  auto xphase = [&](auto role_tag, auto upd_tag, auto sc_tag, auto pre_tag, int uu, int us)
      __attribute__((always_inline)) {
    constexpr int R = decltype(role_tag)::value;
    constexpr bool UPD = decltype(upd_tag)::value, SC = decltype(sc_tag)::value;
    constexpr bool PRE = decltype(pre_tag)::value;
    constexpr int NU = UPD ? 4 * NDB : 0;   // update products (qb, g, db)
    constexpr int NP = NU + (SC ? 2 * NKS : 0);   // then score products (ks, qb), ks-major
    static_assert(!PRE || NU >= PF, "pre-read operands are update operands");
    int lo = 0, hi = 0;
    const __bf16* tu = UPD ? upd_tile(role_tag, uu, lo, hi) : qsm;
    int eb = (us % (R ? 2 : NB)) * TILE;
    int qo = qoff0;
    asm volatile("" : "+s"(eb), "+v"(qo));
    const __bf16* ts = (R ? gsm : qsm) + eb;
    const __bf16* vt = vsm + kgrp * 32 * D;
    bf16x8 a[NP], vb[NKS];
    auto rd = [&](int i) __attribute__((always_inline)) {
      if (i < NU) {
        a[i] = upd_operand(tu, lo, hi, i);
      } else {
        const int ks = (i - NU) >> 1, qb = (i - NU) & 1;
        a[i] = *(const bf16x8*)(ts + qb * 32 * D + (qo ^ (16 * ks)));
        if constexpr (R == 1)
          if (qb == 0) vb[ks] = *(const bf16x8*)(vt + (qo ^ (16 * ks)));
      }
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if constexpr (PRE)
        a[i] = apre[i];
      else
        rd(i);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + PF < NP) rd(i + PF);
      if (i < NU) {
        const int qb = i / (2 * NDB), g = (i / NDB) & 1, db = i % NDB;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], pk[qb][g], acc[db], 0, 0, 0);
      } else {
        const int ks = (i - NU) >> 1, qb = (i - NU) & 1;
        const bf16x8 bop = R ? vb[ks] : bf[ks];
        acc2[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bop, ks == 0 ? f32x16{} : acc2[qb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The packed values are computed in the vector phase: without this the
  // compiler sinks their arithmetic past the barrier into the wave's
  // matrix-core phase, where it cannot overlap the wave's own products.
  auto pin_packed = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(pk[0][0]), "+v"(pk[0][1]), "+v"(pk[1][0]), "+v"(pk[1][1]));
  };
  // register r of block qb holds query q0t + 32 qb + 8 (r/4) + 4 lh + r%4 of
  // key mykey; quarter x = r/4 = 2 g + half.  The vector phases go group by
  // group (qb, g); the P wave reads all its lse values first, the dS wave
  // reads each group's LDS values one group ahead.
  auto p_values = [&](auto masked_tag, int u) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int buf = u % NB;
    const int q0t = (first + u) * BQ;
    // every group's lse is read up front: the partner wave's operand reads
    // keep the LDS queue long, and a read one group ahead stalls each group
    f32x4 lv[4][2];                       // [group][half]
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        lv[gi][half] = *(const f32x4*)&rowv[buf][0][16 * gi + 8 * half + 4 * lh];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {      // gi = 2 qb + g
      const int qb = gi >> 1, g = gi & 1;
      u32x4 w;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int x = 2 * g + half;
        f32x4 pe;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = fast_exp2(__builtin_fmaf(acc2[qb][4 * x + e], c, -lv[gi][half][e]));
          if constexpr (MASKED) {
            const int q = q0t + 16 * gi + 8 * half + 4 * lh + e;
            if (q >= N || (CAUSAL && mykey > q)) v = 0.f;
          }
          pe[e] = v;
        }
        pbuf[kgrp][4 * qb + x][lane] = pe;
        w[2 * half] = pack_bf16x2(pe[0], pe[1]);
        w[2 * half + 1] = pack_bf16x2(pe[2], pe[3]);
      }
      pk[qb][g] = __builtin_bit_cast(bf16x8, w);
      __builtin_amdgcn_sched_barrier(0);
    }
    pin_packed();
  };
  auto ds_values = [&](int u) __attribute__((always_inline)) {
    const int buf = u % NB;
    f32x4 dv4[4][2], pe[4][2];            // [group][half]
    auto rd = [&](int gi) __attribute__((always_inline)) {
      const int qb = gi >> 1, g = gi & 1;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        dv4[gi][half] = *(const f32x4*)&rowv[buf][1][16 * gi + 8 * half + 4 * lh];
        pe[gi][half] = pbuf[kgrp][4 * qb + 2 * g + half][lane];
      }
    };
    rd(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      if (gi + 1 < 4) rd(gi + 1);
      const int qb = gi >> 1, g = gi & 1;
      u32x4 w;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int x = 2 * g + half;
        float dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dsv[e] = pe[gi][half][e] * (acc2[qb][4 * x + e] - dv4[gi][half][e]);
        w[2 * half] = pack_bf16x2(dsv[0], dsv[1]);
        w[2 * half + 1] = pack_bf16x2(dsv[2], dsv[3]);
      }
      pk[qb][g] = __builtin_bit_cast(bf16x8, w);
      __builtin_amdgcn_sched_barrier(0);
    }
    pin_packed();
  };
  // tile u's P needs the mask: causal diagonal (or keys after all its
  // queries) or rows past N
  auto tile_masked = [&](int u) {
    const int q0 = (first + u) * BQ;
    return (q0 + BQ > N) || (CAUSAL && q0 < kw0 + 31);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  using R0 = std::integral_constant<int, 0>;
  using R1 = std::integral_constant<int, 1>;
  // Each loop iteration is one (matrix-core, vector) phase pair, so the
  // accumulators keep their registers from phase to phase.  A vector phase
  // ends by reading the first operands of the wave's next update (its tile
  // is complete: it was awaited before the barrier that began the phase);
  // an empty asm keeps those reads after the phase's LDS writes.
  if (role == 0) {
    // phase 0: S(0); phase 1: P(0); phase 2i+2: dV(i), S(i+1); phase 2i+3: P(i+1)
    phase_begin(0);
    __builtin_amdgcn_s_setprio(3);
    xphase(R0{}, F_{}, T_{}, F_{}, 0, 0);
    __builtin_amdgcn_s_setprio(0);
    phase_end(0);
    phase_begin(1);
    if (tile_masked(0))
      p_values(T_{}, 0);
    else
      p_values(F_{}, 0);
    asm volatile("" ::: "memory");
    pre_read(R0{}, 0);
    phase_end_pre(1);
    for (int i = 0; i + 1 < nt; ++i) {
      phase_begin(2 * i + 2);
      __builtin_amdgcn_s_setprio(3);
      xphase(R0{}, T_{}, T_{}, T_{}, i, i + 1);
      __builtin_amdgcn_s_setprio(0);
      phase_end(2 * i + 2);
      phase_begin(2 * i + 3);
      if (tile_masked(i + 1))
        p_values(T_{}, i + 1);
      else
        p_values(F_{}, i + 1);
      asm volatile("" ::: "memory");
      pre_read(R0{}, i + 1);
      phase_end_pre(2 * i + 3);
    }
    phase_begin(2 * nt);
    xphase(R0{}, T_{}, F_{}, T_{}, nt - 1, 0);
    phase_end(2 * nt);
    phase_begin(2 * nt + 1);
    phase_end(2 * nt + 1);
  } else {
    // phase 0: dP(0); phase 1: -; phase 2i+2: dS(i); phase 2i+3: dK(i), dP(i+1)
    phase_begin(0);
    __builtin_amdgcn_s_setprio(3);
    xphase(R1{}, F_{}, T_{}, F_{}, 0, 0);
    __builtin_amdgcn_s_setprio(0);
    phase_end(0);
    phase_begin(1);
    phase_end(1);
    for (int i = 0; i + 1 < nt; ++i) {
      phase_begin(2 * i + 2);
      ds_values(i);
      asm volatile("" ::: "memory");
      pre_read(R1{}, i);
      phase_end_pre(2 * i + 2);
      phase_begin(2 * i + 3);
      __builtin_amdgcn_s_setprio(3);
      xphase(R1{}, T_{}, T_{}, T_{}, i, i + 1);
      __builtin_amdgcn_s_setprio(0);
      phase_end(2 * i + 3);
    }
    phase_begin(2 * nt);
    ds_values(nt - 1);
    asm volatile("" ::: "memory");
    pre_read(R1{}, nt - 1);
    phase_end_pre(2 * nt);
    phase_begin(2 * nt + 1);
    xphase(R1{}, T_{}, F_{}, T_{}, nt - 1, 0);
    phase_end(2 * nt + 1);
  }

  if (mykey < N) {
    __bf16* dst = (__bf16*)(role ? p.dk : p.dv) + head_base + (long long)mykey * tok;
    store_rows<NDB>(dst, acc, role ? p.scale : 1.f, lh);
  }
  }   // work items
}

// ---------------------------------------------------------------------------
// host-side launch (called by the C ABI in attn_api.cpp)
// ---------------------------------------------------------------------------
// The grid of a kernel with `items` work items: one work-group per item,
// or, for causal calls with more items than the device's `cus` compute
// units (a multiple of 8) and an XCD-aware order, one work-group per
// compute unit looping over the items (item_of_n).  Causal items differ in
// length, and a new work-group starts on a compute unit several
// microseconds after the last one ends; non-causal items are all alike and
// measured slightly faster one work-group per item.
// (Only causal launches loop, so the looping kernels are instantiated with
// LOOP = CAUSAL.)
static int bwd_grid(BwdParams& prm, int items, int cus, bool causal) {
  prm.items = items;
  prm.persist = (causal && cus >= 8 && cus % 8 == 0 && items % 8 == 0 && items > cus) ? 1 : 0;
  return prm.persist ? cus : items;
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(BwdParams prm, int cus, hipStream_t stream) {
  const long long rows = (long long)prm.B * prm.N * prm.H;
  const int grid_delta = (int)((rows + 15) / 16);
  hipError_t e = launch_kernel(attn_bwd_delta_kernel<D>, dim3(grid_delta), dim3(256), stream, prm);
  if (e != hipSuccess) return e;
  int grid = bwd_grid(prm, prm.B * prm.H * prm.n_tiles, cus, CAUSAL);
  e = prm.persist
          ? launch_kernel(attn_bwd_dq_kernel<D, CAUSAL, CAUSAL>, dim3(grid), dim3(512), stream, prm)
          : launch_kernel(attn_bwd_dq_kernel<D, CAUSAL, false>, dim3(grid), dim3(512), stream, prm);
  if (e != hipSuccess) return e;
  if constexpr (D == 128) {
    prm.n_ktiles = (prm.N + 127) / 128;
    grid = bwd_grid(prm, prm.B * prm.H * prm.n_ktiles, cus, CAUSAL);
    return prm.persist ? launch_kernel(attn_bwd_dkdv_pair_kernel<D, CAUSAL, CAUSAL>, dim3(grid),
                                       dim3(512), stream, prm)
                       : launch_kernel(attn_bwd_dkdv_pair_kernel<D, CAUSAL, false>, dim3(grid),
                                       dim3(512), stream, prm);
  } else {
    prm.n_ktiles = prm.n_tiles;
    grid = bwd_grid(prm, prm.B * prm.H * prm.n_ktiles, cus, CAUSAL);
    return prm.persist
               ? launch_kernel(attn_bwd_dkdv_kernel<D, CAUSAL, CAUSAL>, dim3(grid), dim3(512), stream, prm)
               : launch_kernel(attn_bwd_dkdv_kernel<D, CAUSAL, false>, dim3(grid), dim3(512), stream, prm);
  }
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* delta, int B, int H, int N, int d, int causal, float scale,
                           int cus, hipStream_t stream) {
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
  if (d == 128)
    return causal ? launch_bwd_t<128, true>(prm, cus, stream) : launch_bwd_t<128, false>(prm, cus, stream);
  return causal ? launch_bwd_t<64, true>(prm, cus, stream) : launch_bwd_t<64, false>(prm, cus, stream);
}

}  // namespace attn
