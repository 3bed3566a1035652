/*
 * nt — batch-1 decode over block-quantized weights on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libnt.so.  Plain pointers and sizes only.  Unless a comment says
 * otherwise, every pointer argument is DEVICE memory, every call only enqueues
 * work on the given HIP stream (a hipStream_t passed as void*; NULL means the
 * null stream) and returns, and device-side faults surface at the caller's
 * next synchronisation.  The library never synchronises the device.
 *
 * Errors: every int-returning call returns NT_OK (0) or a negative nt_status;
 * on error nothing has been enqueued and nt_last_error() (thread-local)
 * describes the failure.  The one exception is an I/O failure while a file-tier
 * layer is read (nt_stream_layers, nt_decode_token, nt_verify_tokens), which
 * the host can only see mid-call: the file ranges are checked before anything is
 * enqueued, but a read error or a file shrinking during the call returns
 * NT_EHOSTMEM with the layers before that one enqueued (h partly updated).
 *
 * Ownership: the caller owns every buffer (weights, activations, caches,
 * workspaces).  The library allocates nothing on these paths and keeps no
 * pointer after a call returns, except that an nt_streamer keeps its staging
 * pointers and its events until nt_stream_destroy.
 *
 * Sources (the ntransformer pages): ntransformer overview, de.news.hada.io —
 * "Überblick über NTransformer" (GGUF Q4_0, Q8_0, Q4_K_M, Q5_K, Q6_K, F16, F32
 * weights), "Hauptfunktionen" (RoPE, GQA, SwiGLU, RMSNorm, KV cache; SLEP
 * streaming overlapping transfer and compute with double buffering),
 * "Architektur und Codestruktur" (GEMV, RMSNorm, RoPE, SwiGLU, softmax
 * kernels), "Roadmap der Entwicklungsphasen" (F16 KV cache; a public C API is
 * planned but not printed, so these signatures are this library's own);
 * the 70B PCIe P2P article, blog.hotdry.top — §gpu-nvme-direct的实现架构
 * (pinned staging memory, double buffering overlapped on streams),
 * §传统数据路径的性能瓶颈分析 (each token reads every weight).
 */
#ifndef NT_H
#define NT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block formats.  Matrices are rows x cols, stored row-major as rows runs of
 * cols / block_elems consecutive blocks (cols is the contiguous dimension).
 * Byte layouts (little-endian, fp16 = IEEE binary16), GGML's:
 *   NT_Q8_0  34 B / 32 weights : d fp16 @0, q int8[32] @2                  w = d*q
 *   NT_Q4_0  18 B / 32 weights : d fp16 @0, nibbles[16] @2                 w = d*(n-8)
 *            (weight i<16: low nibble of byte i; i>=16: high nibble of byte i-16)
 *   NT_Q4_K 144 B / 256 weights: d @0, dmin @2, 8 x (6-bit scale, 6-bit min) packed in 12 B @4,
 *            nibbles[128] @16                                               w = d*sc*q - dmin*m
 *   NT_Q6_K 210 B / 256 weights: low nibbles[128] @0, 2-bit highs[64] @128, int8 scales[16] @192,
 *            d fp16 @208                                                    w = d*s*(q-32)
 *   NT_Q5_K 176 B / 256 weights: d @0, dmin @2, scales and mins packed as in NT_Q4_K @4,
 *            high bits[32] @16, nibbles[128] @48; the fifth code bit of weight i of sub-block
 *            j = i/32 is bit j of high byte i%32                              w = d*sc*q - dmin*m
 *   NT_F16    2 B / 1 weight   : the weight as IEEE binary16 (GGUF's F16 tensors)
 *   NT_F32    4 B / 1 weight   : the weight as IEEE binary32 (GGUF's F32 tensors)
 * (the overview's format list, "Überblick über NTransformer", names both beside the quant types).
 *   NT_Q4_KT  NT_Q4_K's bytes, each row's superblocks rearranged in tiles of 16 (made by
 *            nt_repack; the same 144 B per 256 weights and the same weights).  Tile t of a row
 *            (superblocks 16t .. 16t+m-1, m = min(16, nsb - 16t), nsb = cols/256) starts at byte
 *            2304t of the row and holds: the m 16-byte headers (bytes 0..15 of each block), then
 *            for j < m, g < 4 in that order the 16 code bytes 32g .. 32g+15 of block j's nibbles,
 *            then the 16 code bytes 32g+16 .. 32g+31.  A wave whose lane 4j+g decodes quarter g
 *            of block j then reads whole 128-byte lines with each of its three 16-byte loads,
 *            which lets the GEMV stream them with the nontemporal policy.  Embedding rows,
 *            nt_dequant, the GEMV and the k-token GEMM (on the vector units) read it;
 *            nt_gemv_q and the layer calls never take the streamed path for it.
 *   NT_Q8_0T  NT_Q8_0's bytes, each row's blocks rearranged in tiles of 64 (made by nt_repack;
 *            34 B per 32 weights, the same weights; cols a multiple of 256 so that rows stay
 *            16-byte multiples).  Tile t of a row (blocks 64t .. 64t+m-1, m = min(64, nb - 64t),
 *            nb = cols/32) starts at byte 2176t and holds, in block order, the first 16 codes of
 *            each block (block bytes 2..17), then the last 16 (bytes 18..33), then the m fp16
 *            scales (bytes 0..1): lane l of a wave reads block l's parts, each load whole lines.
 *            Read where NT_Q4_KT is (register path only, nontemporal loads from 10^8 weights).
 *   NT_Q5_KT  NT_Q5_K's bytes in tiles of 16 superblocks (made by nt_repack; 176 B per 256 weights).
 *            Tile t of a row (m superblocks) starts at byte 2816t and holds the m 16-byte headers
 *            (block bytes 0..15), the m first halves of the high bits (16..31), the m second halves
 *            (32..47), then code bytes 48+32g .. +15 of each (j, g) in lane order, then 64+32g ..
 *            +15 in lane order; read where NT_Q4_KT is.
 * Every entry point that takes cols for NT_F16 / NT_F32 needs a multiple of 32 (so that rows
 * keep the 16-byte alignment the loads use).
 */
typedef enum { NT_Q8_0 = 0, NT_Q4_0 = 1, NT_Q4_K = 2, NT_Q6_K = 3, NT_Q5_K = 4, NT_F16 = 5, NT_F32 = 6,
               NT_Q4_KT = 7, NT_Q8_0T = 8, NT_Q5_KT = 9 } nt_format;

typedef enum {
  NT_OK = 0,
  NT_EINVAL = -1,   /* null pointer, bad count, or inconsistent arguments */
  NT_EFORMAT = -2,  /* unknown format id */
  NT_ESHAPE = -3,   /* size not a multiple of the block, zero/negative, or over a stated limit */
  NT_EALIGN = -4,   /* a pointer is not aligned as its argument requires */
  NT_EHOSTMEM = -5, /* a host buffer that must be page-locked is not */
  NT_EHIP = -6      /* a HIP runtime call failed (message has the HIP error) */
} nt_status;

const char* nt_last_error(void);
const char* nt_version(void);

int nt_block_elems(int fmt);                                /* weights per block, or NT_EFORMAT */
int nt_block_bytes(int fmt);                                /* bytes per block, or NT_EFORMAT */
int64_t nt_matrix_bytes(int fmt, int64_t rows, int64_t cols); /* bytes of a rows x cols matrix, or < 0 */

/* Largest cols accepted by the GEMV entry points (x is held in LDS, padded). */
#define NT_GEMV_MAX_COLS 32768
/* Largest rows (and vocabulary size) accepted anywhere: row and row-group indices stay in
 * 32-bit integer range inside the kernels. */
#define NT_MAX_ROWS (1 << 30)

/* Dequantize a whole matrix to fp32: w[r*cols + c].  Every value equals the
 * block's exact weight rounded once (round-to-nearest-even) to fp32.
 * A test hook for the bit-exactness of the decoders (format pages above).
 * blocks: 4-byte aligned.  Returns NT_ESHAPE if cols % block_elems != 0. */
int nt_dequant(int fmt, int64_t rows, int64_t cols, const void* blocks, float* w, void* stream);

/* Rearrange a Q4_K, Q8_0 or Q5_K matrix (rows x cols, GGUF's block order) into the NT_Q4_KT,
 * NT_Q8_0T or NT_Q5_KT layout above: a layout of the same weights for the GEMV's loads ("Überblick über
 * NTransformer" names the formats; the tiles are this library's own).  fmt: the target layout,
 * NT_Q4_KT (src in NT_Q4_K), NT_Q8_0T (src in NT_Q8_0) or NT_Q5_KT (src in NT_Q5_K), else NT_EFORMAT.  cols: a positive
 * multiple of 256 up to 2^24; rows <= NT_MAX_ROWS (else NT_ESHAPE).  src, dst: device,
 * 16-byte aligned (NT_EALIGN), nt_matrix_bytes(fmt, rows, cols) bytes each, not overlapping
 * (NT_EINVAL; the caller copies back if it wants the matrix in place).  Enqueued on stream;
 * src is only read. */
int nt_repack(int fmt, int64_t rows, int64_t cols, const void* src, void* dst, void* stream);

/* y = W x for a block-quantized W (rows x cols), x and y fp32.
 * The GEMV step of the decode path (ntransformer overview, "Architektur und
 * Codestruktur").  blocks: 16-byte aligned; x: 16-byte aligned, cols floats;
 * y: rows floats, overwritten, must not overlap x or blocks.
 * cols must be a multiple of the block size and <= NT_GEMV_MAX_COLS;
 * rows <= NT_MAX_ROWS.  Accuracy: |y_r - sum_c w_rc x_c| <= 1e-3 * sum_c |w_rc x_c|
 * (fp32 accumulation, scale factors applied per block). */
int nt_gemv_q(int fmt, int64_t rows, int64_t cols, const void* blocks, const float* x, float* y, void* stream);

/* Launch policy of the GEMVs (nt_gemv_q and every GEMV of the layer, token and head calls):
 * a launch whose matrices hold at least min_weights weights in all (rows x cols summed over
 * the matrices it covers) takes the streamed global->LDS path where the formats (Q8_0, Q4_0,
 * Q6_K) and alignment allow it, and so does one of at least min_weights / 8 weights whose
 * register-path waves would each run 7 or more work items in a row (long rows over few row
 * groups, which the streamed path splits over several waves); the others take the register
 * path.  Default 10^8, the measured crossover on MI355X (the streamed path costs more per
 * launch and streams faster).  0 streams every launch the formats allow; a value no launch
 * reaches (say 2^62) keeps every launch on the register path.
 * Both paths compute the same products to the accuracy stated above.  Process-wide, read at
 * every launch: set it while no other host thread enqueues GEMVs.  min_weights < 0 leaves the
 * policy unchanged.  Returns the previous value. */
int64_t nt_set_stream_min_weights(int64_t min_weights);

/* Largest token count of nt_gemm_q. */
#define NT_GEMM_MAX_TOK 8

/* y[t*rows + r] = sum_c W[r][c] x[t*cols + c] for t < n_tok: the GEMV for n_tok tokens
 * at once, reading each weight once.  This is the weight-bound step of the verification
 * pass of self-speculative decoding, where the draft tokens proposed by the VRAM-resident
 * layers meet the whole model in one pass (ntransformer overview, "Hauptfunktionen").
 * 1 <= n_tok <= NT_GEMM_MAX_TOK; x: n_tok x cols fp32, 16-byte aligned; y: n_tok x rows
 * fp32, overwritten, must not overlap x or blocks; blocks: 16-byte aligned; cols a positive
 * multiple of the block size (any width: wide matrices run as several launches over column
 * chunks, each adding into y); rows and cols <= NT_MAX_ROWS.  Per token, the accuracy of nt_gemv_q.
 * Q4_K, Q5_K and Q6_K with 3 to 8 tokens run on the matrix cores (8-bit integer MFMA of activation digits
 * and weight codes, exact in int32); the other cases on the vector ALUs.  A token's outputs
 * do not depend on the other tokens of the call.
 * Errors as nt_gemv_q, and NT_ESHAPE for n_tok out of range; nothing is enqueued then. */
int nt_gemm_q(int fmt, int64_t rows, int64_t cols, int n_tok, const void* blocks, const float* x, float* y,
              void* stream);

/* RMSNorm: y_i = gain_i * x_i / sqrt(mean_j x_j^2 + eps)  (eps inside the root).
 * ntransformer overview, "Hauptfunktionen" (RMSNorm).  y may equal x.  n <= 2^24. */
int nt_rmsnorm(int64_t n, const float* x, const float* gain, float eps, float* y, void* stream);

/* RoPE in place on n_heads consecutive heads of head_dim floats: the adjacent
 * pair (2i, 2i+1) of each head turns by the angle pos * theta^(-2i/head_dim)
 * (angles formed in fp64).  ntransformer overview, "Hauptfunktionen" (RoPE).
 * head_dim even, <= 1024; pos >= 0. */
int nt_rope(int n_heads, int head_dim, int pos, float theta, float* qk, void* stream);

/* KV cache layout (per layer, head_dim 128, fp16 bits, capacity max_ctx slots):
 *   K: [n_kv_heads][max_ctx][128]: element (g, t, d) at (g * max_ctx + t) * 128 + d;
 *   V: groups of 8 slots, [n_kv_heads][max_ctx / 8][128][8]: element (g, t, d) at
 *      g * max_ctx * 128 + ((t / 8) * 128 + d) * 8 + t % 8,
 * so that the 8 consecutive slots of one dimension are one 16-byte piece (the operand
 * shape of the attention's p V product). */
#define NT_MAX_CTX 524288

/* GQA decode attention for one token.  q: [n_q_heads][head_dim] fp32.
 * k_cache, v_cache: fp16 bits in the KV cache layout below.  Query head h
 * reads KV head h / (n_q_heads / n_kv_heads) and attends over cache slots
 * [0, n_ctx): s_t = q.k_t / sqrt(head_dim), p = softmax(s), out_h = sum_t p_t v_t.
 * ntransformer overview, "Hauptfunktionen" (GQA, KV cache) and "Architektur
 * und Codestruktur" (softmax).  out: [n_q_heads][head_dim] fp32.
 * ws: scratch of nt_attn_decode_ws_bytes() bytes, 256-byte aligned, for the
 * per-split partials (two kernels: split partials, then their merge); no initial
 * contents are required.
 * head_dim == 128; n_q_heads % n_kv_heads == 0; n_q_heads / n_kv_heads in
 * {1, 2, 4, 8, 16}; max_ctx a multiple of 8 up to NT_MAX_CTX; 1 <= n_ctx <= max_ctx.
 * Slots at or past n_ctx may hold any bits; they are not used. */
int nt_attn_decode(int n_q_heads, int n_kv_heads, int head_dim, int n_ctx, int max_ctx, const float* q,
                   const uint16_t* k_cache, const uint16_t* v_cache, float* out, void* ws, size_t ws_bytes,
                   void* stream);
size_t nt_attn_decode_ws_bytes(int n_q_heads, int n_kv_heads, int head_dim, int max_ctx);

/* SwiGLU: out_i = gate_i / (1 + exp(-gate_i)) * up_i.
 * ntransformer overview, "Hauptfunktionen" (SwiGLU).  out may equal gate or up. */
int nt_swiglu(int64_t n, const float* gate, const float* up, float* out, void* stream);

/* ------------------------------------------------------------------ layers */

typedef struct {
  int dim;        /* hidden size */
  int n_q_heads;
  int n_kv_heads;
  int head_dim;   /* must be 128 */
  int ffn_dim;
  int max_ctx;    /* cache capacity in slots: a multiple of 8, <= NT_MAX_CTX */
  float eps;      /* RMSNorm epsilon */
  float rope_theta;
} nt_layer_shape;

/* Matrix order in every per-layer array below. */
enum { NT_W_Q = 0, NT_W_K, NT_W_V, NT_W_O, NT_W_GATE, NT_W_UP, NT_W_DOWN, NT_W_COUNT };

typedef struct {
  int fmt[NT_W_COUNT];        /* nt_format of q, k, v, o, gate, up, down */
  const void* w[NT_W_COUNT];  /* device blocks, 16-byte aligned: q [nq*hd x dim], k, v [nkv*hd x dim],
                                 o [dim x nq*hd], gate, up [ffn x dim], down [dim x ffn] */
  const float* attn_norm;     /* [dim] */
  const float* ffn_norm;      /* [dim] */
} nt_layer_weights;

/* One Llama decode layer for the token at position pos (ntransformer overview,
 * "Hauptfunktionen"):
 *   n1 = RMSNorm(h, attn_norm); q = Wq n1, k = Wk n1, v = Wv n1; RoPE(q, k, pos);
 *   k, v -> fp16 (RNE) into cache slot pos; o = attention over slots [0, pos];
 *   h1 = h + Wo o; n2 = RMSNorm(h1, ffn_norm); a = SwiGLU(Wg n2, Wu n2); h2 = h1 + Wd a.
 * h: [dim] fp32, in/out (h2 on return).  k_cache, v_cache: the KV cache layout above.
 * ws: nt_decode_layer_ws_bytes() bytes, 256-byte aligned; no initial contents are required.
 * After the call ws holds, as fp32 arrays
 * at these byte offsets (see nt_decode_layer_ws_offsets): the rotated query q [nq*hd],
 * the attention output o [nq*hd], h1 [dim] and the SwiGLU output a [ffn].
 * Constraints: head_dim 128; dim, nq*hd and ffn multiples of 256 and <= NT_GEMV_MAX_COLS;
 * 0 <= pos < max_ctx; q/k/v share one format family launch (any of the four formats). */
int nt_decode_layer(const nt_layer_weights* w, const nt_layer_shape* shp, int pos, float* h, uint16_t* k_cache,
                    uint16_t* v_cache, void* ws, size_t ws_bytes, void* stream);
size_t nt_decode_layer_ws_bytes(const nt_layer_shape* shp);

/* One decode layer for n_tok tokens at consecutive positions pos .. pos + n_tok - 1 at once:
 * the verification pass of self-speculative decoding, where the draft tokens proposed by the
 * VRAM-resident layers run through the whole model together (ntransformer overview,
 * "Hauptfunktionen": self-speculative decoding; RMSNorm, RoPE, GQA, SwiGLU, KV cache).
 * Token t is the single-token layer of nt_decode_layer at position pos + t: its k and v go to
 * cache slot pos + t, and it attends over slots [0, pos + t] (the earlier draft tokens of the
 * call included, the later ones not).  Each weight matrix is read once for all n_tok tokens
 * (the k-token GEMM of nt_gemm_q; the residual adds accumulate into h).
 * h: [n_tok][dim] fp32, in/out.  1 <= n_tok <= NT_GEMM_MAX_TOK; 0 <= pos, pos + n_tok <= max_ctx.
 * ws: nt_decode_layer_k_ws_bytes() bytes, 256-byte aligned, no initial contents required; after
 * the call it holds, as fp32 [n_tok][...] arrays at the offsets nt_decode_layer_k_ws_offsets
 * gives (q, o, h1, a), each token's rotated query, attention output, h1 and SwiGLU output.
 * Accuracy per token as nt_decode_layer; the results are those of n_tok sequential
 * nt_decode_layer calls up to rounding (n_tok = 1 runs nt_decode_layer's own launches, bit for
 * bit).  Other constraints and errors as nt_decode_layer. */
int nt_decode_layer_k(const nt_layer_weights* w, const nt_layer_shape* shp, int pos, int n_tok, float* h,
                      uint16_t* k_cache, uint16_t* v_cache, void* ws, size_t ws_bytes, void* stream);
size_t nt_decode_layer_k_ws_bytes(const nt_layer_shape* shp, int n_tok);  /* 0 for a bad shape or n_tok */
/* off[0..3] = byte offsets of q, o, h1 and a ([n_tok][...] fp32 each) in that workspace */
int nt_decode_layer_k_ws_offsets(const nt_layer_shape* shp, int n_tok, int64_t* off);

/* Bytes of the static workspace of nt_decode_layer_noalloc (per device). */
#define NT_NOALLOC_WS_BYTES (8 << 20)

/* nt_decode_layer for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same launches, with the
 * workspace taken from a static device array of NT_NOALLOC_WS_BYTES that each device holds
 * until the process ends, found on the first call on a device (with that device current)
 * instead of a caller buffer.  The call allocates nothing.  Shapes whose
 * nt_decode_layer_ws_bytes() exceeds NT_NOALLOC_WS_BYTES are rejected with NT_ESHAPE (the
 * 70B shape at 4224 cache slots needs 0.8 MB; the limit is reached near 60000 slots).  Every
 * call on a device shares that device's array: calls that overlap in time on one device
 * (other streams, other host threads) race on it and must be ordered by the caller.  After
 * the call the array holds the stage outputs nt_decode_layer leaves in its workspace.
 * Arguments, results and errors otherwise as nt_decode_layer. */
int nt_decode_layer_noalloc(const nt_layer_weights* w, const nt_layer_shape* shp, int pos, float* h,
                            uint16_t* k_cache, uint16_t* v_cache, void* stream);

/* The FFN input half of a decode layer on its own, the same launch nt_decode_layer makes:
 * a = SwiGLU(Wg n, Wu n) with n = RMSNorm(h, ffn_norm) (ntransformer overview,
 * "Hauptfunktionen": RMSNorm, SwiGLU).  h: device [dim] fp32, 16-byte aligned, read only;
 * a: device [ffn] fp32.  Same shape and weight constraints as nt_decode_layer (the other
 * matrices of w must be valid pointers but are not read). */
int nt_ffn_up(const nt_layer_weights* w, const nt_layer_shape* shp, const float* h, float* a, void* stream);
/* off[0..4] = byte offsets of q, o, h1, a and the attention partials inside the layer workspace */
int nt_decode_layer_ws_offsets(const nt_layer_shape* shp, int64_t* off);

/* ------------------------------------------------------------ token glue */

/* h = dequantized row *token of an embedding table [n_vocab x dim] (token read on
 * the device).  A token outside [0, n_vocab) writes zeros.  table: 4-byte aligned. */
int nt_embed_row(int fmt, int64_t n_vocab, int64_t dim, const void* table, const int32_t* token, float* h,
                 void* stream);

/* *out_index = first index of the maximum of v[0..n) (greedy pick; ties -> lowest index). */
int nt_argmax(int64_t n, const float* v, int32_t* out_index, void* stream);

/* *out = sum_i a_i b_i / sqrt(sum_i a_i^2 * sum_i b_i^2), or 0 if a or b is all zeros: the
 * cosine similarity of a layer's input and output hidden states, by which cosine-based layer
 * skip ranks layers (ntransformer overview, "Leistung und Caching-Struktur": 20 of 80 layers
 * skipped).  Sums in fp64; |error| below 1e-6.  a, b: device [n], n in [1, 2^24]; out:
 * device, one float.  A calibration pass keeps a copy of h before each layer, runs the
 * layer, and calls this on (copy, h). */
int nt_layer_cosine(int64_t n, const float* a, const float* b, float* out, void* stream);

/* Measurement helper, not a step of the decode: reads `bytes` of device memory at buf with
 * plain 16-byte nontemporal vector loads (32 workgroups of 256 threads per CU, two loads in
 * flight per thread) and discards them, so that the time it takes is the achievable HBM read rate
 * of the part, the yardstick for the GEMVs' rates next to the published peak.  buf: device,
 * 16-byte aligned, bytes a positive multiple of 16; sink: device, 4 bytes, written only in
 * the (never expected) case that the folded data equals a fixed constant.  Errors: NT_ESHAPE,
 * NT_EINVAL, NT_EALIGN, NT_EHIP (nothing enqueued). */
int nt_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* ------------------------------------------------------- models, streaming */

/* Where each tensor of a layer sits in one contiguous layer blob (bytes). */
typedef struct {
  int64_t offset[NT_W_COUNT + 2]; /* q, k, v, o, gate, up, down, attn_norm, ffn_norm; 256-byte aligned */
  int fmt[NT_W_COUNT];
  int64_t blob_bytes;
} nt_layer_layout;

/* Where a layer's blob lives (ntransformer overview, "Leistung und Caching-Struktur": VRAM-
 * resident layers, pinned RAM for H2D transfers, and a file fallback; "Hauptfunktionen": the
 * data path picks the fastest tier that holds the layer). */
enum { NT_TIER_PINNED = 0, NT_TIER_RESIDENT = 1, NT_TIER_FILE = 2 };

typedef struct {
  const void* blob;     /* device pointer if resident, page-locked HOST pointer if pinned, unused for a file */
  int resident;         /* NT_TIER_RESIDENT: run in place; NT_TIER_PINNED: copied from host memory into a
                           staging buffer; NT_TIER_FILE: read from fd at file_offset into the streamer's
                           page-locked bounce buffers, then copied into a staging buffer */
  uint16_t* k_cache;    /* device, fp16, the KV cache layout above */
  uint16_t* v_cache;
  int skip;             /* 1: layer skip: the layer is not run (h passes through unchanged, its
                           cache is not written, a streamed blob is not copied, and its blob,
                           caches and tier are not checked, so a plan whose streamed layers are
                           all skipped runs without a streamer); the caller picks
                           the layers, e.g. those whose nt_layer_cosine of input and output is
                           highest (ntransformer overview, "Leistung und Caching-Struktur") */
  int fd;               /* NT_TIER_FILE: an open file descriptor readable with pread */
  int64_t file_offset;  /* NT_TIER_FILE: byte offset of the blob in that file */
} nt_layer_entry;

typedef struct {
  nt_layer_shape shape;
  nt_layer_layout layout;
  int n_layers;
  const nt_layer_entry* layers; /* host array of n_layers entries */
} nt_model_plan;

typedef struct {
  int64_t layers_streamed;  /* layers that ran from a staging buffer in this call */
  int64_t h2d_bytes;        /* bytes copied host-to-device by this call (prefetches included) */
} nt_stream_stats;

typedef struct nt_streamer nt_streamer;

/* A double-buffered layer streamer (ntransformer overview, "Hauptfunktionen":
 * SLEP overlaps transfer and compute with double buffering; 70B PCIe P2P
 * article, §gpu-nvme-direct的实现架构: pinned staging memory and two buffers on
 * streams).  staging0/1: device buffers of staging_bytes each, 256-byte aligned,
 * owned by the caller.  Creates four HIP events (on the current device). */
int nt_stream_create(void* staging0, void* staging1, size_t staging_bytes, nt_streamer** out);
void nt_stream_destroy(nt_streamer* st);

/* Give a streamer the page-locked host bounce buffers (bounce_bytes each, caller-owned,
 * 4096-byte aligned) that NT_TIER_FILE layers are read into before their H2D copy, and the
 * number of host threads (1..64) that read each blob in parallel pieces with pread.  The
 * three stages of a file layer -- read into a bounce buffer, copy to a staging buffer,
 * compute -- overlap across layers: while the GPU runs layer n, the calling thread reads
 * layer n + 2 (70B PCIe P2P article, §gpu-nvme-direct的实现架构: a three-stage pipeline;
 * here through the page cache, without the raw-device path). */
int nt_stream_set_bounce(nt_streamer* st, void* bounce0, void* bounce1, size_t bounce_bytes, int n_threads);

/* Run all plan->n_layers layers for the token at pos over h (in/out, [dim]).
 * Resident layers run in place on `compute`.  A streamed layer's blob is copied
 * by hipMemcpyAsync on `copy` into a free staging buffer as soon as that buffer
 * frees (the compute stream records "free" events, the copy stream "ready"
 * events), so copies run ahead of compute and across calls: at the end of a
 * call the first streamed layers of the next token are already in flight.
 * Pinned blobs must be page-locked host memory (NT_EHOSTMEM otherwise); file layers need
 * bounce buffers (nt_stream_set_bounce; NT_EINVAL otherwise), and a short or failed read is
 * NT_EHOSTMEM.  Every streamed blob must fit staging_bytes.  ws as for nt_decode_layer.  compute != copy.  stats nullable.
 * A streamer must be used with one plan at a time, from one host thread.  The copies it
 * prefetches at the end of a call are used by the next call only if the plan's entries
 * still name the same sources (blob, or file and offset); otherwise they are drained and
 * the sequence restarts. */
int nt_stream_layers(nt_streamer* st, const nt_model_plan* plan, int pos, float* h, void* ws, size_t ws_bytes,
                     void* compute, void* copy, nt_stream_stats* stats);

typedef struct {
  int embd_fmt;
  const void* token_embd;   /* device [n_vocab x dim] blocks */
  int64_t n_vocab;
  const float* output_norm; /* device [dim] */
  int out_fmt;
  const void* output;       /* device [n_vocab x dim] blocks (LM head) */
} nt_model_head;

/* One greedy decode token: h = embed(*token); all layers (nt_stream_layers, or in
 * place when st is NULL, which requires every layer resident); logits =
 * W_out RMSNorm(h, output_norm); *token = argmax(logits) (ties -> lowest id).
 * token: device int32, in/out.  logits: device [n_vocab] fp32.  h: device [dim].
 * ws: nt_decode_token_ws_bytes() bytes, 256-byte aligned; no initial contents are required. */
int nt_decode_token(nt_streamer* st, const nt_model_plan* plan, const nt_model_head* head, int pos, int32_t* token,
                    float* logits, float* h, void* ws, size_t ws_bytes, void* compute, void* copy,
                    nt_stream_stats* stats);
size_t nt_decode_token_ws_bytes(const nt_layer_shape* shp);

/* The verification pass of self-speculative decoding over the whole model (ntransformer
 * overview, "Hauptfunktionen": the draft tokens of the VRAM-resident layers are checked by the
 * full model in one pass): the n_tok input tokens tokens[t] at positions pos + t run through
 * every layer of the plan together (nt_decode_layer_k; streamed layers as in nt_stream_layers,
 * each blob copied once for all tokens), then the final RMSNorm and the LM head for every
 * token (the k-token GEMM), and next[t] = the greedy pick after token t (first index of the
 * largest logit).  A caller that drafted tokens[1..] from tokens[0] accepts the draft tokens
 * while tokens[t + 1] == next[t], and continues from the first next[t] that differs.
 * tokens, next: device int32[n_tok]; logits: device [n_tok][n_vocab] fp32; h: device
 * [n_tok][dim] fp32 (the final hidden states on return).  ws: nt_verify_tokens_ws_bytes()
 * bytes, 256-byte aligned.  1 <= n_tok <= NT_GEMM_MAX_TOK; pos + n_tok <= max_ctx.
 * Other arguments, constraints and errors as nt_decode_token. */
int nt_verify_tokens(nt_streamer* st, const nt_model_plan* plan, const nt_model_head* head, int pos, int n_tok,
                     const int32_t* tokens, int32_t* next, float* logits, float* h, void* ws, size_t ws_bytes,
                     void* compute, void* copy, nt_stream_stats* stats);
size_t nt_verify_tokens_ws_bytes(const nt_layer_shape* shp, int n_tok);

/* Workspace bytes of nt_lm_head (the packed argmax key). */
#define NT_LM_HEAD_WS_BYTES 256

/* The greedy head on its own, the same launches nt_decode_token ends with (ntransformer
 * overview, "Architektur und Codestruktur": the sampler after the model; "Hauptfunktionen":
 * RMSNorm): logits = W_out RMSNorm(h, output_norm) with W_out an n_vocab x dim block
 * matrix (the GEMV, its RMSNorm prologue and a fused argmax epilogue in one launch), then
 * *token = the first index of the largest logit (ties -> lowest index; a NaN logit never
 * wins).  h: device [dim] fp32, 16-byte aligned, read only; output: 16-byte aligned blocks;
 * output_norm: device [dim], 16-byte aligned; logits: device [n_vocab] fp32, overwritten;
 * token: device int32.  ws: NT_LM_HEAD_WS_BYTES bytes, 256-byte aligned, no initial contents
 * required.  dim a positive multiple of 256 up to NT_GEMV_MAX_COLS; 1 <= n_vocab <= NT_MAX_ROWS.
 * Errors: NT_EFORMAT, NT_ESHAPE, NT_EINVAL (null pointer, eps < 0, workspace too small),
 * NT_EALIGN, NT_EHIP; nothing is enqueued then. */
int nt_lm_head(int fmt, int64_t n_vocab, int64_t dim, const void* output, const float* output_norm, float eps,
               const float* h, float* logits, int32_t* token, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- measurement hook */

/* Kernel classes that can be timed with HIP events recorded around each launch
 * on the launching stream (adds small gaps; for measurement runs only).  The first
 * five are the launches of a decode layer, NT_K_LM_HEAD the LM head of
 * nt_decode_token / nt_model_head; NT_K_ATTN also covers nt_attn_decode and
 * NT_K_GEMV covers nt_gemv_q, NT_K_GEMM nt_gemm_q (one interval per call). */
enum { NT_K_ATTN_IN = 0, NT_K_ATTN, NT_K_O, NT_K_FFN_UP, NT_K_FFN_DOWN, NT_K_LM_HEAD, NT_K_GEMV, NT_K_GEMM, NT_K_COUNT };
/* Start timing launches of kernel class kclass (one class at a time); up to
 * max_launches launches are recorded.  Creates events on the current device. */
int nt_timing_begin(int kclass, int max_launches);
/* Wait for the recorded launches, return their count and summed milliseconds, and stop timing. */
int nt_timing_end(int* n_launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* NT_H */
