/*
 * oracle.c — plain, slow, obviously-correct CPU reference for paged KV cache
 * decode.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the bench's
 * CPU-baseline leg call it; the product path never does.  It shares no code,
 * header, table or helper with the HIP library; it is written from the
 * pool-layout definition and from the pages below.
 *
 * Pages followed:
 *   [P1] "LLM inference basics and vLLM internals" (ttlab.hopto.org):
 *        §2 (KV cache holds K and V of every past token; bytes per token
 *        2*L*H_kv*d*b; GQA groups query heads onto one KV head; FP8 KV makes
 *        b = 1), §4 (fixed-size blocks, default 16 tokens; per-request table
 *        from logical to physical block; shared prefix blocks; block 0 is
 *        the reserved null block).
 *   [P2] "vLLM internals (2): why PagedAttention pages the KV cache"
 *        (youngju.dev), "Block table" (logical block j -> physical block id;
 *        the kernel finds blocks through the table).
 *   [P4] "vToken" (gotosocial.chinng-lab-srv.dev), "KV cache basics" (only
 *        the new token's K/V are computed and appended).
 *
 * Floating point: every attention quantity is fp64.  The fp8 encoder works
 * on the fp32 value x*inv (one IEEE fp32 multiply), then picks the nearest
 * E4M3 value by exhaustive search over the decoded code table.
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (never -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 0, ORC_FP16 = 1, ORC_FP8 = 2 };

/* ------------------------------------------------------------ sizes ---- */

/* [P1] §2: bytes per token = 2 (K and V) * layers * kv heads * head dim *
 * element bytes. */
int64_t orc_bytes_per_token(int64_t layers, int64_t kv_heads, int64_t head_dim,
                            int64_t elem_bytes) {
    return 2 * layers * kv_heads * head_dim * elem_bytes;
}

static int elem_bytes(int dtype) { return dtype == ORC_FP8 ? 1 : 2; }

/* ----------------------------------------------------------- codecs ---- */

/* bfloat16 is the upper 16 bits of an IEEE binary32. */
double orc_bf16_value(uint16_t bits) {
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_fp16_value(uint16_t bits) {
    int sign = bits >> 15;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);               /* subnormal */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25); /* 1.frac * 2^(e-15) */
    return sign ? -v : v;
}

/* OCP OFP8 E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
 * is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity, so
 * S.1111.110 = 448 is the largest finite value. */
double orc_e4m3_value(uint8_t code) {
    int sign = code >> 7;
    int expo = (code >> 3) & 0xf;
    int mant = code & 0x7;
    double v;
    if (expo == 15 && mant == 7)
        return NAN;
    if (expo == 0)
        v = ldexp((double)mant, -9);
    else
        v = ldexp((double)(8 + mant), expo - 10);    /* 1.m * 2^(e-7) */
    return sign ? -v : v;
}

void orc_e4m3_table(double* out256) {
    for (int c = 0; c < 256; ++c) out256[c] = orc_e4m3_value((uint8_t)c);
}

/* Round an fp32 value to E4M3: nearest finite value, ties to the even code
 * (mantissa LSB 0), magnitudes beyond 448 saturate to 448, NaN stays NaN,
 * the sign is kept (also for results that round to zero). */
uint8_t orc_e4m3_encode(float x) {
    if (isnan(x)) return (uint8_t)(signbit(x) ? 0xff : 0x7f);
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (a >= 448.0) return (uint8_t)(sign | 0x7e);   /* saturate (incl. inf) */
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7e; ++c) {          /* every finite magnitude */
        double err = fabs(orc_e4m3_value((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1))) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(sign | best);
}

void orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i]);
}

static double elem_value(const uint8_t* p, int dtype) {
    if (dtype == ORC_FP8) return orc_e4m3_value(p[0]);
    uint16_t bits = (uint16_t)(p[0] | (p[1] << 8));   /* little endian */
    return dtype == ORC_BF16 ? orc_bf16_value(bits) : orc_fp16_value(bits);
}

/* ----------------------------------------------------------- layout ---- */

/* Byte offset of element (row r, dim k) inside a 16-token sub-tile, K pool.
 * Eight consecutive dims of one token form a group; group c of token r goes
 * to lane r + 16*(c%4) of 1 KiB row c/4 (two groups share a lane slot when
 * elements are one byte). */
int64_t orc_k_sub_offset(int r, int k, int eb) {
    int c = k / 8, e = k % 8;
    int lane = r + 16 * (c % 4);
    int kk = c / 4;
    int per_slot = 2 / eb;
    return 1024LL * (kk / per_slot) + 16 * lane + 8 * eb * (kk % per_slot) + eb * e;
}

/* V pool: four consecutive tokens of one dim form a group; the group of dim
 * k, tokens 4*(r/4).., goes to lane k%16 + 16*(r/4) of 1 KiB row
 * (k/16)/per_slot. */
int64_t orc_v_sub_offset(int r, int k, int eb) {
    int nt = k / 16, i = r % 4;
    int lane = (k % 16) + 16 * (r / 4);
    int per_slot = 4 / eb;
    return 1024LL * (nt / per_slot) + 16 * lane + 4 * eb * (nt % per_slot) + eb * i;
}

/* Byte offset of (physical block pb, kv head g, token row t of the block,
 * dim k) in a pool of [num_blocks][kv_heads] tiles of block_size x d. */
int64_t orc_pool_offset(int64_t pb, int g, int t, int k, int is_value,
                        int kv_heads, int head_dim, int block_size, int dtype) {
    int eb = elem_bytes(dtype);
    int64_t tile = (int64_t)block_size * head_dim * eb;
    int64_t sub = 16LL * head_dim * eb;
    int64_t base = (pb * kv_heads + g) * tile + (t / 16) * sub;
    return base + (is_value ? orc_v_sub_offset(t % 16, k, eb)
                            : orc_k_sub_offset(t % 16, k, eb));
}

/* --------------------------------------------------------- indexing ---- */

/* [P1] §4 / [P2] "Block table": the token at logical position pos of a
 * sequence lives in physical block table[pos / bs] at row pos % bs; its slot
 * number is that block * bs + row. */
int64_t orc_slot_of_position(const int32_t* table_row, int pos, int block_size) {
    return (int64_t)table_row[pos / block_size] * block_size + pos % block_size;
}

/* Slot of every sequence's newest token (position c-1), -1 if c <= 0 or the
 * position lies past the table. */
void orc_decode_slots(const int32_t* block_tables, int max_blocks, const int32_t* ctx,
                      int num_seqs, int block_size, int64_t* slots) {
    for (int s = 0; s < num_seqs; ++s) {
        int c = ctx[s];
        if (c <= 0 || c > max_blocks * block_size) {
            slots[s] = -1;
            continue;
        }
        slots[s] = orc_slot_of_position(block_tables + (int64_t)s * max_blocks, c - 1,
                                        block_size);
    }
}

/* ---------------------------------------------------- cache writing ---- */

/* Write each new token's K/V rows into the pools in place ([P4] "KV cache
 * basics": only new tokens are added).  src: [T][kv_heads][d] raw 16-bit
 * values of src_dtype.  bf16/fp16 pools take the bits unchanged; an fp8
 * pool takes encode(fp32(x) * inv_scale), inv_scale = fp32(1 / scale).
 * Slots < 0 or >= num_blocks*bs are skipped. */
void orc_reshape_and_cache(const uint16_t* key, const uint16_t* value, int src_dtype,
                           uint8_t* k_pool, uint8_t* v_pool, const int64_t* slots,
                           int num_tokens, int kv_heads, int head_dim, int block_size,
                           int64_t num_blocks, int kv_dtype, float k_scale,
                           float v_scale) {
    float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
    for (int t = 0; t < num_tokens; ++t) {
        int64_t slot = slots[t];
        if (slot < 0 || slot >= num_blocks * block_size) continue;
        int64_t pb = slot / block_size;
        int row = (int)(slot % block_size);
        for (int g = 0; g < kv_heads; ++g) {
            for (int k = 0; k < head_dim; ++k) {
                int64_t src = ((int64_t)t * kv_heads + g) * head_dim + k;
                for (int which = 0; which < 2; ++which) {
                    uint16_t bits = which ? value[src] : key[src];
                    uint8_t* pool = which ? v_pool : k_pool;
                    int64_t off = orc_pool_offset(pb, g, row, k, which, kv_heads,
                                                  head_dim, block_size, kv_dtype);
                    if (kv_dtype == ORC_FP8) {
                        float x = (float)(src_dtype == ORC_BF16 ? orc_bf16_value(bits)
                                                                : orc_fp16_value(bits));
                        float xs = x * (which ? v_inv : k_inv);
                        pool[off] = orc_e4m3_encode(xs);
                    } else {
                        pool[off] = (uint8_t)(bits & 0xff);
                        pool[off + 1] = (uint8_t)(bits >> 8);
                    }
                }
            }
        }
    }
}

/* ------------------------------------------------- decode attention ---- */

/* out[s][h][:] = sum_t softmax_t(scale * q[s][h] . K_t) V_t over the c_s
 * tokens reached through block_tables[s] ([P1] §4, [P2] "Block table"),
 * with kv head g = h / G for G = heads / kv_heads ([P1] §2, GQA), all in
 * fp64.  fp8 pools dequantise as code * scale.  c <= 0 gives zeros.
 * q: [S][heads][d] raw 16-bit values of q_dtype.  out: [S][heads][d] fp64.
 * Runs (s, h) pairs in parallel when OpenMP is available. */
void orc_paged_decode(double* out, const uint16_t* q, int q_dtype, const uint8_t* k_pool,
                      const uint8_t* v_pool, int kv_dtype, const int32_t* block_tables,
                      int max_blocks, const int32_t* ctx, int num_seqs, int heads,
                      int kv_heads, int head_dim, int block_size, float scale,
                      float k_scale, float v_scale) {
    int group = heads / kv_heads;
    double kdq = kv_dtype == ORC_FP8 ? (double)k_scale : 1.0;
    double vdq = kv_dtype == ORC_FP8 ? (double)v_scale : 1.0;
    int64_t pairs = (int64_t)num_seqs * heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t sh = 0; sh < pairs; ++sh) {
        int s = (int)(sh / heads), h = (int)(sh % heads), g = h / group;
        double* o = out + sh * head_dim;
        for (int k = 0; k < head_dim; ++k) o[k] = 0.0;
        int c = ctx[s];
        if (c <= 0) continue;
        const int32_t* row = block_tables + (int64_t)s * max_blocks;
        double* qd = malloc(sizeof(double) * head_dim);
        double* logit = malloc(sizeof(double) * c);
        for (int k = 0; k < head_dim; ++k) {
            uint16_t bits = q[sh * head_dim + k];
            qd[k] = q_dtype == ORC_BF16 ? orc_bf16_value(bits) : orc_fp16_value(bits);
        }
        double mx = -INFINITY;
        for (int t = 0; t < c; ++t) {
            int64_t pb = row[t / block_size];
            double dot = 0.0;
            for (int k = 0; k < head_dim; ++k) {
                int64_t off = orc_pool_offset(pb, g, t % block_size, k, 0, kv_heads,
                                              head_dim, block_size, kv_dtype);
                dot += qd[k] * (elem_value(k_pool + off, kv_dtype) * kdq);
            }
            logit[t] = (double)scale * dot;
            if (logit[t] > mx) mx = logit[t];
        }
        double denom = 0.0;
        for (int t = 0; t < c; ++t) {
            double w = exp(logit[t] - mx);
            denom += w;
            int64_t pb = row[t / block_size];
            for (int k = 0; k < head_dim; ++k) {
                int64_t off = orc_pool_offset(pb, g, t % block_size, k, 1, kv_heads,
                                              head_dim, block_size, kv_dtype);
                o[k] += w * (elem_value(v_pool + off, kv_dtype) * vdq);
            }
        }
        for (int k = 0; k < head_dim; ++k) o[k] /= denom;
        free(qd);
        free(logit);
    }
}

/* Multi-token attention over the paged cache ([P1] §5/§6: the tokens of a
 * prefill chunk, or those left after a prefix-cache hit, are the last
 * q_len tokens of their sequence; each attends to every earlier token and
 * itself).  For query row r of sequence s (rows query_start[s] ..
 * query_start[s+1]-1), token j = r - query_start[s] sits at position
 * p = c - q_len + j and its output is the softmax-weighted sum over keys
 * t = 0 .. p, read through the block table as in orc_paged_decode.  A row
 * with p < 0 is zero.  Written out directly: one row, one head at a time. */
void orc_paged_prefill(double* out, const uint16_t* q, int q_dtype, const uint8_t* k_pool,
                       const uint8_t* v_pool, int kv_dtype, const int32_t* block_tables,
                       int max_blocks, const int32_t* ctx, const int32_t* query_start,
                       int num_seqs, int heads, int kv_heads, int head_dim, int block_size,
                       float scale, float k_scale, float v_scale) {
    int group = heads / kv_heads;
    double kdq = kv_dtype == ORC_FP8 ? (double)k_scale : 1.0;
    double vdq = kv_dtype == ORC_FP8 ? (double)v_scale : 1.0;
    int64_t rows = query_start[num_seqs];
    int64_t pairs = rows * heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t rh = 0; rh < pairs; ++rh) {
        int64_t r = rh / heads;
        int h = (int)(rh % heads), g = h / group;
        int s = 0;
        while (query_start[s + 1] <= r) ++s;           /* the sequence owning row r */
        int q_len = query_start[s + 1] - query_start[s];
        int j = (int)(r - query_start[s]);
        int c = ctx[s];
        int pos = c - q_len + j;
        double* o = out + rh * head_dim;
        for (int k = 0; k < head_dim; ++k) o[k] = 0.0;
        if (pos < 0) continue;
        int n = pos + 1;                               /* keys 0 .. pos */
        const int32_t* row = block_tables + (int64_t)s * max_blocks;
        double* qd = malloc(sizeof(double) * head_dim);
        double* logit = malloc(sizeof(double) * n);
        for (int k = 0; k < head_dim; ++k) {
            uint16_t bits = q[rh * head_dim + k];
            qd[k] = q_dtype == ORC_BF16 ? orc_bf16_value(bits) : orc_fp16_value(bits);
        }
        double mx = -INFINITY;
        for (int t = 0; t < n; ++t) {
            int64_t pb = row[t / block_size];
            double dot = 0.0;
            for (int k = 0; k < head_dim; ++k) {
                int64_t off = orc_pool_offset(pb, g, t % block_size, k, 0, kv_heads,
                                              head_dim, block_size, kv_dtype);
                dot += qd[k] * (elem_value(k_pool + off, kv_dtype) * kdq);
            }
            logit[t] = (double)scale * dot;
            if (logit[t] > mx) mx = logit[t];
        }
        double denom = 0.0;
        for (int t = 0; t < n; ++t) {
            double w = exp(logit[t] - mx);
            denom += w;
            int64_t pb = row[t / block_size];
            for (int k = 0; k < head_dim; ++k) {
                int64_t off = orc_pool_offset(pb, g, t % block_size, k, 1, kv_heads,
                                              head_dim, block_size, kv_dtype);
                o[k] += w * (elem_value(v_pool + off, kv_dtype) * vdq);
            }
        }
        for (int k = 0; k < head_dim; ++k) o[k] /= denom;
        free(qd);
        free(logit);
    }
}

/* Decode through a per-token table ("vToken" page, "the core idea:
 * token-level virtualisation"): logical token t of sequence s sits at
 * physical slot token_slots[s][t] (block slot / block_size, row slot %
 * block_size), whatever the order of the slots; the result is the same
 * softmax attention over the c = ctx[s] logical tokens as orc_paged_decode,
 * whose block table is the special case slot = table[t / bs] * bs + t % bs. */
void orc_paged_decode_tokens(double* out, const uint16_t* q, int q_dtype, const uint8_t* k_pool,
                             const uint8_t* v_pool, int kv_dtype, const int32_t* token_slots,
                             int max_tokens, const int32_t* ctx, int num_seqs, int heads,
                             int kv_heads, int head_dim, int block_size, float scale,
                             float k_scale, float v_scale) {
    int group = heads / kv_heads;
    double kdq = kv_dtype == ORC_FP8 ? (double)k_scale : 1.0;
    double vdq = kv_dtype == ORC_FP8 ? (double)v_scale : 1.0;
    int64_t pairs = (int64_t)num_seqs * heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t sh = 0; sh < pairs; ++sh) {
        int s = (int)(sh / heads), h = (int)(sh % heads), g = h / group;
        double* o = out + sh * head_dim;
        for (int k = 0; k < head_dim; ++k) o[k] = 0.0;
        int c = ctx[s];
        if (c <= 0) continue;
        const int32_t* slots = token_slots + (int64_t)s * max_tokens;
        double* qd = malloc(sizeof(double) * head_dim);
        double* logit = malloc(sizeof(double) * c);
        for (int k = 0; k < head_dim; ++k) {
            uint16_t bits = q[sh * head_dim + k];
            qd[k] = q_dtype == ORC_BF16 ? orc_bf16_value(bits) : orc_fp16_value(bits);
        }
        double mx = -INFINITY;
        for (int t = 0; t < c; ++t) {
            int64_t pb = slots[t] / block_size;
            int row = slots[t] % block_size;
            double dot = 0.0;
            for (int k = 0; k < head_dim; ++k) {
                int64_t off = orc_pool_offset(pb, g, row, k, 0, kv_heads, head_dim, block_size,
                                              kv_dtype);
                dot += qd[k] * (elem_value(k_pool + off, kv_dtype) * kdq);
            }
            logit[t] = (double)scale * dot;
            if (logit[t] > mx) mx = logit[t];
        }
        double denom = 0.0;
        for (int t = 0; t < c; ++t) {
            double w = exp(logit[t] - mx);
            denom += w;
            int64_t pb = slots[t] / block_size;
            int row = slots[t] % block_size;
            for (int k = 0; k < head_dim; ++k) {
                int64_t off = orc_pool_offset(pb, g, row, k, 1, kv_heads, head_dim, block_size,
                                              kv_dtype);
                o[k] += w * (elem_value(v_pool + off, kv_dtype) * vdq);
            }
        }
        for (int k = 0; k < head_dim; ++k) o[k] /= denom;
        free(qd);
        free(logit);
    }
}

/* Move whole tokens ("vToken" page, asynchronous repacking: a surviving
 * token's K and V move to another slot, the logical order is kept by the
 * token table): for each (src, dst) slot pair, every element of every kv
 * head of the token's K and V rows is copied, in every layer's pools given.
 * All sources are read before any destination is written. */
void orc_move_tokens(uint8_t* const* k_pools, uint8_t* const* v_pools, int num_layers,
                     const int32_t* moves, int num_moves, int kv_heads, int head_dim,
                     int block_size, int kv_dtype) {
    int e = kv_dtype == ORC_FP8 ? 1 : 2;
    size_t per = (size_t)kv_heads * head_dim * e;
    uint8_t* tmp = malloc(per * 2 * (size_t)(num_moves > 0 ? num_moves : 1));
    for (int l = 0; l < num_layers; ++l) {
        for (int pass = 0; pass < 2; ++pass) {
            for (int i = 0; i < num_moves; ++i) {
                int32_t slot = moves[2 * i + pass];           /* pass 0 reads src, pass 1 writes dst */
                int64_t pb = slot / block_size;
                int row = slot % block_size;
                for (int which = 0; which < 2; ++which) {
                    uint8_t* pool = which ? v_pools[l] : k_pools[l];
                    uint8_t* t = tmp + ((size_t)i * 2 + which) * per;
                    for (int g = 0; g < kv_heads; ++g)
                        for (int k = 0; k < head_dim; ++k) {
                            int64_t off = orc_pool_offset(pb, g, row, k, which, kv_heads,
                                                          head_dim, block_size, kv_dtype);
                            uint8_t* x = t + ((size_t)g * head_dim + k) * e;
                            for (int b = 0; b < e; ++b) {
                                if (pass == 0) x[b] = pool[off + b];
                                else pool[off + b] = x[b];
                            }
                        }
                }
            }
        }
    }
    free(tmp);
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
