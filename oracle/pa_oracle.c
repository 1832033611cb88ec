/*
 * pa_oracle.c -- plain, slow, fp64 CPU oracle for the paged KV-cache write and
 * single-query paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the HIP library; it depends on
 * libc and libm only.
 *
 * What it follows:
 *  - "vLLM: Easy, Fast, and Cheap LLM Serving with PagedAttention" (Hacker News
 *    thread), comments contrasting FlashAttention with PagedAttention: both
 *    compute exact attention; paging only changes where keys and values live.
 *    So the decode result is the plain definition out = softmax(scale*q.K^T).V
 *    over the logical tokens 0..L-1 of the sequence, written out here.
 *  - "vLLM Project Update" talk transcript, PagedAttention recap: attention that
 *    works on fixed-size blocks of the KV cache, with per-sequence
 *    logical->physical block maps managed like virtual memory pages.
 *  - "vLLM Project Update" talk transcript, roadmap: multi-query attention
 *    kernels for speculative decoding, where several proposed tokens of one
 *    sequence are scored in one pass; each of them attends causally to the
 *    context up to its own position (orc_decode_mq).
 *  - "[core] Multi Step Scheduling" pull request (vllm-project/vllm #7000),
 *    review thread on ops.advance_step: the per-step GPU state is a slot
 *    mapping, per-sequence block tables, sequence lengths and a block size.
 *
 * Storage convention shared with the GPU library (a format both sides must
 * agree on, not arithmetic).  Tokens of a block are kept in quads of four
 * consecutive offsets; X = 16 / element bytes (8 for the 16-bit types, 4 for
 * fp32):
 *   key cache   [num_blocks][num_kv_heads][block_size/4][head_dim/X][4][X]
 *               (key element e of the token at offset o: quad o/4, chunk e/X,
 *               row o%4, lane e%X)
 *   value cache [num_blocks][num_kv_heads][block_size/4][head_dim][4]
 *               (value element e of offset o: quad o/4, dim e, row o%4)
 *   slot s -> block s / block_size, offset s % block_size.
 *
 * Every floating-point step is done in double precision.  Half, bfloat16 and
 * E4M3 inputs are decoded from their bit patterns by their definitions (sign,
 * biased exponent, significand), not by any hardware conversion; E4M3 caches
 * carry one scale per tensor (stored value * scale = cache element).  The softmax is the two-pass form: max, then exp/sum, so its
 * arithmetic differs on purpose from an online (streaming) softmax.
 *
 * Parity pins (tests/test_oracle.py): contiguous brute force in numpy, the
 * half/bfloat16 decoders against numpy/torch over all 65536 patterns, a
 * E4M3 decoder (all 256 patterns) and encoder (random values, the format's
 * ties, subnormals and saturation) against torch's float8_e4m3fn and the
 * format's definition, hand-worked cache-write layout fixtures (16-bit, fp32
 * and E4M3 with scales), block-permutation and block-size
 * invariance, L=1 -> V, identical keys -> mean(V), one-hot probe -> V[t*],
 * scale 0 -> mean(V), GQA == replicated MHA; the advance step against a
 * hand-worked table and against the seeded generator's own slot arithmetic.
 * No function here is unpinned.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2
#define ORC_FP8 3 /* 8-bit float, OCP E4M3 (cache storage only) */

#define ORC_OK 0
#define ORC_ERR_ARG -1
#define ORC_ERR_SLOT -2
#define ORC_ERR_BLOCK -3
#define ORC_ERR_LEN -4
#define ORC_ERR_MEM -5

/* ---- element decoding --------------------------------------------------- */

/* IEEE-754 binary16: 1 sign, 5 exponent (bias 15), 10 significand bits. */
double orc_f16_bits_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (expo == 0) {
    v = ldexp((double)man, -24); /* subnormal: man * 2^(1-15-10) */
  } else if (expo == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexp((double)(man + 1024), expo - 25); /* (1.man) * 2^(expo-15) */
  }
  return sign ? -v : v;
}

/* bfloat16: the upper half of an IEEE-754 binary32: 1 sign, 8 exponent
 * (bias 127), 7 significand bits. */
double orc_bf16_bits_to_double(uint16_t b) {
  int sign = (b >> 15) & 1;
  int expo = (b >> 7) & 0xff;
  int man = b & 0x7f;
  double v;
  if (expo == 0) {
    v = ldexp((double)man, -133); /* subnormal: man * 2^(1-127-7) */
  } else if (expo == 255) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexp((double)(man + 128), expo - 134); /* (1.man) * 2^(expo-127) */
  }
  return sign ? -v : v;
}

/* IEEE-754 binary32 decoded the same way (1/8/23). */
double orc_f32_bits_to_double(uint32_t f) {
  int sign = (f >> 31) & 1;
  int expo = (f >> 23) & 0xff;
  uint32_t man = f & 0x7fffffu;
  double v;
  if (expo == 0) {
    v = ldexp((double)man, -149);
  } else if (expo == 255) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexp((double)(man + 0x800000u), expo - 150);
  }
  return sign ? -v : v;
}

/* OCP 8-bit floating point, E4M3 variant: 1 sign, 4 exponent (bias 7) and 3
 * significand bits; no infinities; the patterns S.1111.111 are NaN, so the
 * largest finite magnitude is 1.75 * 2^8 = 448; exponent field 0 holds the
 * subnormals man * 2^-9. */
double orc_fp8_e4m3_bits_to_double(uint8_t c) {
  int sign = (c >> 7) & 1;
  int expo = (c >> 3) & 0xf;
  int man = c & 0x7;
  double v;
  if (expo == 15 && man == 7) {
    v = NAN;
  } else if (expo == 0) {
    v = ldexp((double)man, -9);
  } else {
    v = ldexp((double)(man + 8), expo - 10); /* (1.man) * 2^(expo-7) */
  }
  return sign ? -v : v;
}

/* A float as E4M3: the representable value nearest to y, ties to the even
 * significand; magnitudes beyond 448 (infinities included) give +-448
 * (saturation); NaN gives the NaN pattern with y's sign. */
uint8_t orc_fp8_e4m3_from_float(float y) {
  const uint8_t sign = signbit(y) ? 0x80 : 0x00;
  if (isnan(y)) return sign | 0x7f;
  const double a = fabs((double)y);
  if (a >= 448.0) return sign | 0x7e;
  /* spacing of the representable magnitudes around a */
  double spacing;
  if (a < ldexp(1.0, -6)) {
    spacing = ldexp(1.0, -9);
  } else {
    int e2;
    frexp(a, &e2); /* a = f * 2^e2 with f in [0.5, 1), so 2^(e2-1) <= a */
    spacing = ldexp(1.0, e2 - 1 - 3);
  }
  const double n = nearbyint(a / spacing); /* default rounding: nearest, ties even */
  const double r = n * spacing;
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -6)) return sign | (uint8_t)n; /* subnormal: significand n */
  int e2;
  const double f = frexp(r, &e2); /* r = (2f) * 2^(e2-1), 2f in [1, 2) */
  const int expo = e2 - 1 + 7;
  const int man = (int)((2.0 * f - 1.0) * 8.0);
  return sign | (uint8_t)(expo << 3) | (uint8_t)man;
}

/* 65536-entry decode tables, each entry produced by the decoder above; they
 * only save the repeated ldexp calls on large inputs. */
static double g_f16_table[65536];
static double g_bf16_table[65536];
static double g_fp8_table[256];
static pthread_once_t g_tables_once = PTHREAD_ONCE_INIT;

static void orc_fill_tables(void) {
  for (uint32_t i = 0; i < 65536; ++i) {
    g_f16_table[i] = orc_f16_bits_to_double((uint16_t)i);
    g_bf16_table[i] = orc_bf16_bits_to_double((uint16_t)i);
  }
  for (uint32_t i = 0; i < 256; ++i) g_fp8_table[i] = orc_fp8_e4m3_bits_to_double((uint8_t)i);
}

static int orc_elem_bytes(int dtype) {
  switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_FP8: return 1;
    default: return 0;
  }
}

/* Element idx of an array of the given dtype, as a double. */
static double orc_load(const void* base, int dtype, int64_t idx) {
  if (dtype == ORC_F32) {
    uint32_t bits;
    memcpy(&bits, (const char*)base + idx * 4, 4);
    return orc_f32_bits_to_double(bits);
  }
  if (dtype == ORC_FP8) return g_fp8_table[((const uint8_t*)base)[idx]];
  uint16_t bits;
  memcpy(&bits, (const char*)base + idx * 2, 2);
  return dtype == ORC_F16 ? g_f16_table[bits] : g_bf16_table[bits];
}

/* ---- cache write (reshape-and-cache) ------------------------------------ */

/*
 * For every token i with slot_mapping[i] >= 0, copy its key row and value
 * row, for every kv head, into the slot's physical block, as raw bits.
 * Tokens are applied in increasing i.  A negative slot means "skip" (padding).
 * k is read at k[i*k_token_stride + h*head_dim + e]; likewise v.
 * Returns ORC_ERR_SLOT (and stops) on a slot >= num_blocks*block_size.
 */
int orc_cache_write(const void* k, const void* v, const int64_t* slot_mapping,
                    int64_t num_tokens, int64_t k_token_stride,
                    int64_t v_token_stride, void* k_cache, void* v_cache,
                    int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                    int32_t block_size, int32_t dtype) {
  int eb = orc_elem_bytes(dtype);
  if (!eb || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || num_tokens < 0 || head_dim % (16 / eb) != 0 || block_size % 4 != 0)
    return ORC_ERR_ARG;
  const int64_t H = num_kv_heads, D = head_dim, BS = block_size, X = 16 / eb;
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    if (slot >= num_blocks * BS) return ORC_ERR_SLOT;
    int64_t blk = slot / BS;
    int64_t off = slot % BS;
    for (int64_t h = 0; h < H; ++h) {
      for (int64_t e = 0; e < D; ++e) {
        int64_t src_k = i * k_token_stride + h * D + e;
        int64_t src_v = i * v_token_stride + h * D + e;
        int64_t quad = (blk * H + h) * (BS / 4) + off / 4;
        int64_t dst_k = ((quad * (D / X) + e / X) * 4 + off % 4) * X + e % X;
        int64_t dst_v = (quad * D + e) * 4 + off % 4;
        memcpy((char*)k_cache + dst_k * eb, (const char*)k + src_k * eb, eb);
        memcpy((char*)v_cache + dst_v * eb, (const char*)v + src_v * eb, eb);
      }
    }
  }
  return ORC_OK;
}

/*
 * The same write into E4M3 caches with per-tensor scales ("vLLM Project
 * Update" talk, quantization update: the engine keeps the KV cache in 8-bit
 * floating point; the talk fixes no format or scaling, the reading taken here
 * is OCP E4M3 with one scale per cache tensor): every element x of k (v),
 * read as src_dtype, is stored as e4m3(float(x / k_scale)), the quotient
 * rounded once to float and then to E4M3 as orc_fp8_e4m3_from_float does.
 * The caches use the layout above with X = 16.
 */
int orc_cache_write_fp8(const void* k, const void* v, const int64_t* slot_mapping,
                        int64_t num_tokens, int64_t k_token_stride, int64_t v_token_stride,
                        uint8_t* k_cache, uint8_t* v_cache, int32_t num_kv_heads,
                        int32_t head_dim, int64_t num_blocks, int32_t block_size,
                        int32_t src_dtype, float k_scale, float v_scale) {
  if (!orc_elem_bytes(src_dtype) || src_dtype == ORC_FP8 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || num_blocks <= 0 || num_tokens < 0 ||
      head_dim % 16 != 0 || block_size % 4 != 0 || !(k_scale > 0.0f) || !(v_scale > 0.0f))
    return ORC_ERR_ARG;
  pthread_once(&g_tables_once, orc_fill_tables);
  const int64_t H = num_kv_heads, D = head_dim, BS = block_size, X = 16;
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    if (slot >= num_blocks * BS) return ORC_ERR_SLOT;
    int64_t blk = slot / BS;
    int64_t off = slot % BS;
    for (int64_t h = 0; h < H; ++h) {
      for (int64_t e = 0; e < D; ++e) {
        double xk = orc_load(k, src_dtype, i * k_token_stride + h * D + e);
        double xv = orc_load(v, src_dtype, i * v_token_stride + h * D + e);
        int64_t quad = (blk * H + h) * (BS / 4) + off / 4;
        k_cache[((quad * (D / X) + e / X) * 4 + off % 4) * X + e % X] =
            orc_fp8_e4m3_from_float((float)(xk / (double)k_scale));
        v_cache[(quad * D + e) * 4 + off % 4] =
            orc_fp8_e4m3_from_float((float)(xv / (double)v_scale));
      }
    }
  }
  return ORC_OK;
}

/* ---- decode attention --------------------------------------------------- */

typedef struct {
  double* out;
  const void* q;
  int32_t q_dtype;
  const void* k_cache;
  const void* v_cache;
  int32_t kv_dtype;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
  int32_t num_queries; /* query tokens per sequence */
  int64_t num_blocks;
  int32_t block_size, max_blocks_per_seq;
  double scale;
  double k_scale, v_scale; /* cache element = stored value * scale */
  const int64_t* rows; /* b*num_q_heads + hq, or NULL for all rows */
  int64_t n_rows;
  int32_t n_threads;
  int32_t thread_id;
  int status;
} orc_decode_job;

/*
 * One output row (b, i, hq): out[e] = sum_t w_t v_t[e] / sum_t w_t with
 * s_t = scale * sum_e q[e] k_t[e], m = max_t s_t, w_t = exp(s_t - m),
 * t over the logical positions 0..L-1, K/V rows found through the block
 * table: position t lives in physical block block_tables[b][t / bs] at
 * offset t % bs.  q head hq reads kv head hq / (Hq / Hkv).  With Q query
 * tokens per sequence (the last Q positions of its context_lens[b] tokens),
 * query i sits at position context_lens[b] - Q + i and attends to the
 * positions up to its own: L = context_lens[b] - Q + i + 1.  Q = 1 is plain
 * decode.
 */
static int orc_decode_row(const orc_decode_job* J, int64_t row) {
  const int64_t Hq = J->num_q_heads, Hkv = J->num_kv_heads, D = J->head_dim;
  const int64_t Q = J->num_queries;
  const int64_t X = 16 / orc_elem_bytes(J->kv_dtype);
  const int64_t BS = J->block_size, MB = J->max_blocks_per_seq;
  const int64_t b = row / (Q * Hq), i = (row / Hq) % Q, hq = row % Hq;
  const int64_t group = Hq / Hkv;
  const int64_t hk = hq / group;
  const int64_t Lseq = J->context_lens[b];
  if (Lseq < Q || Lseq > MB * BS) return ORC_ERR_LEN;
  const int64_t L = Lseq - Q + i + 1;

  double* s = (double*)malloc((size_t)L * sizeof(double));
  double* acc = (double*)malloc((size_t)D * sizeof(double));
  if (!s || !acc) {
    free(s);
    free(acc);
    return ORC_ERR_MEM;
  }

  /* scores */
  for (int64_t t = 0; t < L; ++t) {
    int64_t phys = J->block_tables[b * MB + t / BS];
    if (phys < 0 || phys >= J->num_blocks) {
      free(s);
      free(acc);
      return ORC_ERR_BLOCK;
    }
    const int64_t o = t % BS;
    const int64_t quad = (phys * Hkv + hk) * (BS / 4) + o / 4;  // this token's quad
    double dot = 0.0;
    for (int64_t e = 0; e < D; ++e)
      dot += orc_load(J->q, J->q_dtype, row * D + e) *
             (orc_load(J->k_cache, J->kv_dtype, ((quad * (D / X) + e / X) * 4 + o % 4) * X + e % X) *
              J->k_scale);
    s[t] = J->scale * dot;
  }

  /* two-pass softmax: max, then weights and their sum (increasing t) */
  double m = s[0];
  for (int64_t t = 1; t < L; ++t)
    if (s[t] > m) m = s[t];
  double z = 0.0;
  for (int64_t t = 0; t < L; ++t) {
    s[t] = exp(s[t] - m);
    z += s[t];
  }

  /* weighted sum of value rows */
  for (int64_t e = 0; e < D; ++e) acc[e] = 0.0;
  for (int64_t t = 0; t < L; ++t) {
    int64_t phys = J->block_tables[b * MB + t / BS];
    int64_t o = t % BS;
    int64_t quad = (phys * Hkv + hk) * (BS / 4) + o / 4;
    for (int64_t e = 0; e < D; ++e) {
      int64_t vidx = (quad * D + e) * 4 + o % 4;
      acc[e] += s[t] * (orc_load(J->v_cache, J->kv_dtype, vidx) * J->v_scale);
    }
  }
  for (int64_t e = 0; e < D; ++e) J->out[row * D + e] = acc[e] / z;

  free(s);
  free(acc);
  return ORC_OK;
}

static void* orc_decode_worker(void* arg) {
  orc_decode_job* J = (orc_decode_job*)arg;
  int64_t total =
      J->rows ? J->n_rows : (int64_t)J->num_seqs * J->num_queries * J->num_q_heads;
  for (int64_t i = J->thread_id; i < total; i += J->n_threads) {
    int64_t row = J->rows ? J->rows[i] : i;
    int st = orc_decode_row(J, row);
    if (st != ORC_OK) {
      J->status = st;
      break;
    }
  }
  return NULL;
}

/*
 * Decode attention for all rows (rows == NULL) or for the listed rows
 * (row = (b*num_queries + i)*num_q_heads + hq).  q and out are
 * [num_seqs][num_queries][num_q_heads][head_dim]; out is double and only
 * computed rows are written.  Rows are independent, so they are spread over
 * n_threads POSIX threads; each row's arithmetic is sequential.
 */
int orc_decode_mq(double* out, const void* q, int32_t q_dtype, const void* k_cache,
                  const void* v_cache, int32_t kv_dtype,
                  const int32_t* block_tables, const int32_t* context_lens,
                  int32_t num_seqs, int32_t num_queries, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                  int32_t block_size, int32_t max_blocks_per_seq, float scale, float k_scale,
                  float v_scale, const int64_t* rows, int64_t n_rows, int32_t n_threads) {
  if (num_queries < 1) return ORC_ERR_ARG;
  if (!orc_elem_bytes(q_dtype) || q_dtype == ORC_FP8 || !orc_elem_bytes(kv_dtype))
    return ORC_ERR_ARG;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || block_size % 4 != 0 ||
      head_dim % (16 / orc_elem_bytes(kv_dtype)) != 0)
    return ORC_ERR_ARG;
  if (rows) {
    for (int64_t i = 0; i < n_rows; ++i)
      if (rows[i] < 0 || rows[i] >= (int64_t)num_seqs * num_queries * num_q_heads)
        return ORC_ERR_ARG;
  }
  pthread_once(&g_tables_once, orc_fill_tables);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;

  orc_decode_job jobs[256];
  pthread_t tids[256];
  for (int i = 0; i < n_threads; ++i) {
    orc_decode_job* J = &jobs[i];
    J->out = out;
    J->q = q;
    J->q_dtype = q_dtype;
    J->k_cache = k_cache;
    J->v_cache = v_cache;
    J->kv_dtype = kv_dtype;
    J->block_tables = block_tables;
    J->context_lens = context_lens;
    J->num_seqs = num_seqs;
    J->num_q_heads = num_q_heads;
    J->num_kv_heads = num_kv_heads;
    J->num_queries = num_queries;
    J->head_dim = head_dim;
    J->num_blocks = num_blocks;
    J->block_size = block_size;
    J->max_blocks_per_seq = max_blocks_per_seq;
    J->scale = (double)scale;
    J->k_scale = (double)k_scale;
    J->v_scale = (double)v_scale;
    J->rows = rows;
    J->n_rows = n_rows;
    J->n_threads = n_threads;
    J->thread_id = i;
    J->status = ORC_OK;
  }
  if (n_threads == 1) {
    orc_decode_worker(&jobs[0]);
    return jobs[0].status;
  }
  int started = 0;
  for (int i = 0; i < n_threads; ++i) {
    if (pthread_create(&tids[i], NULL, orc_decode_worker, &jobs[i]) != 0) break;
    ++started;
  }
  /* any thread that failed to start: run its share here */
  for (int i = started; i < n_threads; ++i) orc_decode_worker(&jobs[i]);
  for (int i = 0; i < started; ++i) pthread_join(tids[i], NULL);
  for (int i = 0; i < n_threads; ++i)
    if (jobs[i].status != ORC_OK) return jobs[i].status;
  return ORC_OK;
}

/* Single-query decode: orc_decode_mq with one query token per sequence. */
int orc_decode(double* out, const void* q, int32_t q_dtype, const void* k_cache,
               const void* v_cache, int32_t kv_dtype,
               const int32_t* block_tables, const int32_t* context_lens,
               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
               int32_t head_dim, int64_t num_blocks, int32_t block_size,
               int32_t max_blocks_per_seq, float scale, float k_scale, float v_scale,
               const int64_t* rows, int64_t n_rows, int32_t n_threads) {
  return orc_decode_mq(out, q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens,
                       num_seqs, 1, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                       max_blocks_per_seq, scale, k_scale, v_scale, rows, n_rows, n_threads);
}

/* ---- advance step ------------------------------------------------------- */

/*
 * One decode step forward for every live sequence ("[core] Multi Step
 * Scheduling" pull request, review thread on ops.advance_step): the sampled
 * id becomes the next input token, the position moves one forward, the
 * sequence length becomes position + 1, and the slot is the position's offset
 * inside the block the table names (-1 when the table has no block there).
 * Rows num_queries..num_seqs-1 are padding: their slot becomes -1.
 */
int orc_advance_step(int32_t num_seqs, int32_t num_queries, int32_t block_size,
                     int64_t* input_tokens, const int64_t* sampled_token_ids,
                     int64_t* input_positions, int32_t* seq_lens, int64_t* slot_mapping,
                     const int32_t* block_tables, int32_t max_blocks_per_seq) {
  if (num_seqs < 0 || num_queries < 0 || num_queries > num_seqs || block_size <= 0 ||
      max_blocks_per_seq <= 0)
    return ORC_ERR_ARG;
  for (int64_t i = 0; i < num_seqs; ++i) {
    if (i >= num_queries) {
      slot_mapping[i] = -1;
      continue;
    }
    input_tokens[i] = sampled_token_ids[i];
    int64_t position = input_positions[i] + 1;
    input_positions[i] = position;
    seq_lens[i] = (int32_t)(position + 1);
    int64_t logical_block = position / block_size;
    int64_t slot = -1;
    if (logical_block < max_blocks_per_seq) {
      int64_t physical = block_tables[i * max_blocks_per_seq + logical_block];
      if (physical >= 0) slot = physical * block_size + position % block_size;
    }
    slot_mapping[i] = slot;
  }
  return ORC_OK;
}

/* Encoder exposed in bulk for the pins: out[i] = e4m3(y[i]). */
void orc_encode_fp8(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_e4m3_from_float(y[i]);
}

/* Decoders exposed in bulk for the pins: out[i] = decode(bits[i]). */
void orc_decode_bits(const void* bits, int32_t dtype, int64_t n, double* out) {
  pthread_once(&g_tables_once, orc_fill_tables);
  for (int64_t i = 0; i < n; ++i) out[i] = orc_load(bits, dtype, i);
}
