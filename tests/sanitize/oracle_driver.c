/*
 * Sanitizer driver for the CPU oracle (test infrastructure): built together
 * with oracle/tms_oracle.c under -fsanitize=address,undefined and run by
 * tests/test_sanitize.py.  It drives every oracle entry point over seeded
 * random catalogs (prefix pairs, shared prefixes, ragged lengths, both
 * placements of the control ids, fp32 and bf16 tables) and the rejected
 * inputs, so that an out-of-bounds access, a leak or undefined behaviour in
 * the oracle fails the run.  It prints "ok <cases>" and exits 0 when every
 * decode also met the answer invariants checked here (status, exactly k
 * distinct entries, length = sum of entry lengths + k).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct orc_trie orc_trie;
typedef struct orc_state orc_state;
int orc_trie_build(const int32_t*, const int64_t*, int32_t, int32_t, int32_t, int32_t, orc_trie**);
void orc_trie_free(orc_trie*);
void orc_trie_info(const orc_trie*, int32_t*);
void orc_trie_csr(const orc_trie*, int32_t*, int32_t*, int32_t*, int32_t*, int32_t*);
orc_state* orc_state_new(const orc_trie*, int32_t);
void orc_state_free(orc_state*);
int32_t orc_state_legal(const orc_state*, int32_t*, int32_t*);
int32_t orc_state_advance(orc_state*, int32_t);
void orc_state_info(const orc_state*, int32_t*);
void orc_state_live(const orc_state*, int32_t*);
void orc_state_entries(const orc_state*, int32_t*);
double orc_logit(const void*, int, int32_t, int32_t, const void*, double*);
void orc_dense_logits(const void*, int, int32_t, int32_t, const void*, double*);
int orc_decode(const orc_trie*, int32_t, const void*, int, int32_t, int32_t, const void*, int32_t, int32_t,
               const int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, double*, double*, double*, int32_t*);

/* xorshift64* generator: this test program's own seeded draws */
static uint64_t g_rng = 88172645463325252ull;
static uint64_t rnd(void) {
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return g_rng * 2685821657736338717ull;
}
static int32_t rnd_below(int32_t n) { return (int32_t)(rnd() % (uint64_t)n); }

static int fail(const char* what, int c) {
  fprintf(stderr, "case %d: %s\n", c, what);
  return 1;
}

int main(void) {
  int cases = 0;
  for (int c = 0; c < 2000; ++c) {
    const int32_t V = 8 + rnd_below(300);
    const int32_t sep = (c & 1) ? V - 2 : 1, stop = (c & 1) ? V - 1 : 3;
    const int32_t K = 1 + rnd_below(40);
    const int32_t maxlen = 1 + rnd_below(7);
    const int32_t idr = 2 + rnd_below(V - 4 < 12 ? V - 4 : 12); /* small id range: shared prefixes */
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (K + 1));
    int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)K * maxlen + 1);
    off[0] = 0;
    for (int32_t i = 0; i < K; ++i) {
      int32_t len = 1 + rnd_below(maxlen);
      if (i > 0 && rnd_below(4) == 0) { /* a prefix pair: extend the previous entry */
        int32_t pl = (int32_t)(off[i] - off[i - 1]);
        if (pl < maxlen) {
          memcpy(tok + off[i], tok + off[i - 1], sizeof(int32_t) * pl);
          tok[off[i] + pl] = 4 + rnd_below(idr);
          off[i + 1] = off[i] + pl + 1;
          continue;
        }
      }
      for (int32_t j = 0; j < len; ++j) tok[off[i] + j] = 4 + rnd_below(idr); /* never sep or stop (< 4) */
      if (sep > 3) /* ids 4.. may reach V-2: keep them below */
        for (int32_t j = 0; j < len; ++j) tok[off[i] + j] %= (V - 2);
      for (int32_t j = 0; j < len; ++j) if (tok[off[i] + j] < 4) tok[off[i] + j] += 4;
      off[i + 1] = off[i] + len;
    }
    orc_trie* t = NULL;
    int rc = orc_trie_build(tok, off, K, V, sep, stop, &t);
    if (rc != 0) { /* duplicates are rejected: fine, nothing to decode */
      if (t) return fail("handle returned with an error", c);
      free(off);
      free(tok);
      continue;
    }
    int32_t info[8];
    orc_trie_info(t, info);
    const int32_t N = info[0], E = info[1], cap = info[3], md = info[4];
    int32_t *b = malloc(4 * (N + 1)), *en = malloc(4 * N), *tk = malloc(4 * (E ? E : 1)), *ch = malloc(4 * (E ? E : 1)),
            *l0 = malloc(4 * (E ? E : 1));
    orc_trie_csr(t, b, en, tk, ch, l0);
    if (b[N] != E) return fail("edge count", c);
    const int32_t k = 1 + rnd_below(K < 4 ? K : 4);
    const int32_t H = 1 + rnd_below(40);
    const int dtype = (int)(c % 2);
    const int32_t B = 1 + rnd_below(4);
    const int32_t T = k * (md + 1) + rnd_below(3);
    const size_t esz = dtype == 0 ? 4 : 2;
    void* emb = malloc(esz * (size_t)V * H);
    void* hid = malloc(esz * (size_t)T * B * H);
    for (size_t i = 0; i < (size_t)V * H; ++i) {
      const float f = (float)((int64_t)rnd_below(2001) - 1000) / 1000.0f;
      if (dtype == 0) ((float*)emb)[i] = f;
      else { uint32_t u; memcpy(&u, &f, 4); ((uint16_t*)emb)[i] = (uint16_t)(u >> 16); }
    }
    for (size_t i = 0; i < (size_t)T * B * H; ++i) {
      const float f = (float)((int64_t)rnd_below(2001) - 1000) / 500.0f;
      if (dtype == 0) ((float*)hid)[i] = f;
      else { uint32_t u; memcpy(&u, &f, 4); ((uint16_t*)hid)[i] = (uint16_t)(u >> 16); }
    }
    int32_t *out_tok = malloc(4 * (size_t)B * T), *len = malloc(4 * B), *ent = malloc(4 * (size_t)B * k),
            *status = malloc(4 * B), *nl = malloc(4 * (size_t)B * T);
    double *best = malloc(8 * (size_t)B * T), *margin = malloc(8 * (size_t)B * T), *sa = malloc(8 * (size_t)B * T);
    rc = orc_decode(t, k, emb, dtype, V, H, hid, B, T, NULL, out_tok, len, ent, status, best, margin, sa, nl);
    if (rc != 0) return fail("decode", c);
    for (int32_t s = 0; s < B; ++s) {
      if (status[s] != 0) return fail("status", c);
      int32_t sum = 0;
      for (int32_t j = 0; j < k; ++j) {
        if (ent[s * k + j] < 0 || ent[s * k + j] >= K) return fail("entry range", c);
        for (int32_t i = 0; i < j; ++i) if (ent[s * k + i] == ent[s * k + j]) return fail("repeat", c);
        sum += (int32_t)(off[ent[s * k + j] + 1] - off[ent[s * k + j]]);
      }
      if (len[s] != sum + k) return fail("length", c);
    }
    /* teacher-forced along the decode's own tokens: the same answers */
    int32_t* out2 = malloc(4 * (size_t)B * T);
    rc = orc_decode(t, k, emb, dtype, V, H, hid, B, T, out_tok, out2, len, ent, status, NULL, NULL, NULL, NULL);
    if (rc != 0 || memcmp(out2, out_tok, 4 * (size_t)B * T) != 0) return fail("follow", c);
    /* state walk with every call, and a refused token */
    orc_state* st = orc_state_new(t, k);
    int32_t* lt = malloc(4 * (cap ? cap : 1));
    int32_t* le = malloc(4 * (cap ? cap : 1));
    int32_t* lv = malloc(4 * (E ? E : 1));
    int32_t si[6], se[64];
    for (int32_t step = 0; step < T + 1; ++step) {
      const int32_t n = orc_state_legal(st, lt, le);
      orc_state_info(st, si);
      orc_state_live(st, lv);
      orc_state_entries(st, se);
      if (n <= 0) break;
      if (orc_state_advance(st, -5) == 0) return fail("invalid token accepted", c);
      orc_state_free(st);
      st = orc_state_new(t, k);
      for (int32_t r = 0; r < step; ++r) orc_state_advance(st, out_tok[r]);
      orc_state_advance(st, lt[rnd_below(n)]);
      break;
    }
    double* dl = malloc(8 * (size_t)V);
    orc_dense_logits(emb, dtype, V, H, hid, dl);
    double a;
    if (fabs(orc_logit(emb, dtype, H, V - 1, hid, &a) - dl[V - 1]) != 0.0) return fail("logit", c);
    free(dl); free(lt); free(le); free(lv); free(out2);
    orc_state_free(st);
    free(out_tok); free(len); free(ent); free(status); free(nl); free(best); free(margin); free(sa);
    free(emb); free(hid); free(b); free(en); free(tk); free(ch); free(l0);
    orc_trie_free(t);
    free(off);
    free(tok);
    ++cases;
  }
  /* rejected inputs */
  {
    int64_t off[3] = {0, 1, 1};
    int32_t tok[2] = {5, 6};
    orc_trie* t = NULL;
    if (orc_trie_build(tok, off, 2, 16, 14, 15, &t) == 0 || t) return fail("empty entry accepted", -1);
    int64_t off2[2] = {0, 2};
    int32_t tok2[2] = {5, 14};
    if (orc_trie_build(tok2, off2, 1, 16, 14, 15, &t) == 0 || t) return fail("sep inside entry accepted", -1);
  }
  printf("ok %d\n", cases);
  return 0;
}
