/*
 * Plain CPU oracle for the trie-constrained sparse decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product links, loads or calls this
 * file; only the tests, the smoke check and the bench's CPU-baseline leg do.
 * It shares no code with the HIP library (its own trie build, its own state,
 * its own arithmetic) and is written to be checked by eye, not to be fast:
 * scalar loops, fp64 arithmetic, no blocking and no reordering.
 *
 * What it computes (sources: "Constraint made cheaper than no constraint",
 * sections "The grammar as a trie over tokens", "Masked sampling inside the
 * sampler" and "The sparse output layer"; "Constrained decoding with weighted
 * automata", the definition of the next-token mask; "Understanding inference
 * for systems engineers", section 3.8 on the greedy tie rule):
 *
 *   A catalog C is K distinct non-empty token strings over [0,V) without the
 *   separator id sep and the stop id stop.  The answer language is
 *       L_k(C) = { c_p1 sep c_p2 sep ... sep c_pk stop : p an injection [k]->[K] },
 *   i.e. exactly k pointers, none repeated.  After an emitted prefix u the legal
 *   set is Mask(u) = { v : some w makes u v w a string of L_k(C) }.  Each step the
 *   decoder takes the legal token with the largest logit <h_t, E_v>, ties to
 *   the lower token id, and stops after the stop token.
 *
 * The trie form of that definition (token-id trie in CSR, sentinel children for
 * the two control edges, per-edge live counts decremented along a completed
 * pointer's path, a per-terminal spent flag) is written out below in the
 * order the first page describes it.  Readings where the pages are silent:
 *   - control edges are ordinary edges of a terminal's range, labelled sep and
 *     stop, with sentinel children -1 (sep) and -2 (stop);
 *   - the live count of a content edge starts at the number of entries whose
 *     string passes through it (the entry ending at its child included);
 *   - completing a pointer decrements every content edge on its root path and
 *     sets the spent flag of its terminal, which removes both control edges of
 *     that terminal only;
 *   - sep is legal at an unspent terminal iff done+1 < k, stop iff done+1 == k;
 *   - logits are fp64 sums of exact products in index order, never rounded to
 *     bf16 before the argmax; no scale, temperature or softcap.
 *
 * Planted mistakes (negative controls) are selected by orc_set_mutant(); the
 * default 0 is the oracle proper.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* status codes, same numbering as the library's public header */
enum {
  ORC_OK = 0,
  ORC_ERR_INVALID_ARG = 1,
  ORC_ERR_CATALOG = 2,
  ORC_ERR_FANOUT = 3,
  ORC_ERR_K = 4,
  ORC_ERR_EMPTY_MASK = 5,
  ORC_ERR_NOT_WALKABLE = 6,
  ORC_ERR_NOT_DONE = 7,
};

#define CHILD_SEP (-1)
#define CHILD_STOP (-2)

/* planted mistakes for negative-control tests */
enum {
  MUT_NONE = 0,
  MUT_TIE_HIGHER_ID = 1,    /* ties go to the higher token id */
  MUT_NO_LIVE_DECREMENT = 2,/* completing a pointer does not touch live counts */
  MUT_NO_SPENT_FLAG = 3,    /* finished terminals keep their control edges */
  MUT_ROW_OFF_BY_ONE = 4,   /* logit of token v is read from row v+1 */
  MUT_SEP_STOP_SWAPPED = 5, /* sep when the last pointer is due, stop otherwise */
  MUT_DROP_LAST_TERM = 6,   /* dot product skips the last hidden element */
  MUT_MARGIN_ZERO = 7,      /* the top-two margin is reported as 0 */
  MUT_SUMABS_WINNER = 8,    /* sum|p| is the winner's, not the larger of the top two */
  MUT_FOLLOW_IGNORED = 9,   /* teacher forcing advances by the oracle's own pick */
  MUT_CS_FIRST_BYTE = 10,   /* character catalogs: a token is legal when its first byte continues a string */
  MUT_CS_STOP_LEAF_ONLY = 11, /* character catalogs: stop only where no longer string continues */
};
static int g_mutant = 0;
void orc_set_mutant(int m) { g_mutant = m; }

/* ------------------------------------------------------------------------- */
/* Trie build                                                                 */
/* ------------------------------------------------------------------------- */

/* pointer-style build trie: each node keeps an unsorted child list */
typedef struct {
  int32_t *ctok, *cnode; /* child tokens and child build-node ids */
  int32_t nchild, capchild;
  int32_t entry;         /* catalog index ending here, or -1 */
} bnode;

typedef struct {
  int32_t n_nodes, n_edges, n_entries, cap, max_depth, sep, stop, vocab;
  int32_t *begin;  /* [n_nodes+1] edge range of each node */
  int32_t *entry;  /* [n_nodes] catalog index ending at the node, or -1 */
  int32_t *tok;    /* [n_edges] edge label */
  int32_t *child;  /* [n_edges] child node, or -1 (sep) / -2 (stop) */
  int32_t *live0;  /* [n_edges] entries below a content edge; 0 for control */
} orc_trie;

static int32_t bnode_find(const bnode* n, int32_t t) {
  for (int32_t i = 0; i < n->nchild; ++i)
    if (n->ctok[i] == t) return n->cnode[i];
  return -1;
}

static void bnode_add(bnode* n, int32_t t, int32_t id) {
  if (n->nchild == n->capchild) {
    n->capchild = n->capchild ? 2 * n->capchild : 4;
    n->ctok = (int32_t*)realloc(n->ctok, sizeof(int32_t) * n->capchild);
    n->cnode = (int32_t*)realloc(n->cnode, sizeof(int32_t) * n->capchild);
  }
  n->ctok[n->nchild] = t;
  n->cnode[n->nchild] = id;
  n->nchild++;
}

/* insertion sort of a node's children by token (fan-outs are small) */
static void bnode_sort(bnode* n) {
  for (int32_t i = 1; i < n->nchild; ++i) {
    int32_t t = n->ctok[i], c = n->cnode[i], j = i - 1;
    while (j >= 0 && n->ctok[j] > t) {
      n->ctok[j + 1] = n->ctok[j];
      n->cnode[j + 1] = n->cnode[j];
      --j;
    }
    n->ctok[j + 1] = t;
    n->cnode[j + 1] = c;
  }
}

/* number of entries ending at or below build node b (iterative post-order) */
static void count_terminals(const bnode* nodes, int32_t nb, int32_t* below) {
  /* children always get larger build ids than their parent (they are created
   * after it), so a reverse sweep over ids visits children first */
  for (int32_t b = nb - 1; b >= 0; --b) {
    int32_t s = nodes[b].entry >= 0 ? 1 : 0;
    for (int32_t i = 0; i < nodes[b].nchild; ++i) s += below[nodes[b].cnode[i]];
    below[b] = s;
  }
}

void orc_trie_free(orc_trie* t) {
  if (!t) return;
  free(t->begin); free(t->entry); free(t->tok); free(t->child); free(t->live0);
  free(t);
}

/* Validate the catalog and build the canonical CSR: nodes numbered breadth
 * first from root 0 with children in ascending token order; a node's range
 * holds its content edges and, when it is terminal, the sep and stop edges,
 * all in ascending token order. */
int orc_trie_build(const int32_t* tokens, const int64_t* offsets, int32_t K, int32_t vocab,
                   int32_t sep, int32_t stop, orc_trie** out) {
  *out = NULL;
  if (K < 1 || vocab < 2 || sep < 0 || sep >= vocab || stop < 0 || stop >= vocab || sep == stop)
    return ORC_ERR_INVALID_ARG;
  if (offsets[0] != 0) return ORC_ERR_CATALOG;
  for (int32_t i = 0; i < K; ++i) {
    if (offsets[i + 1] <= offsets[i]) return ORC_ERR_CATALOG; /* empty entry */
    for (int64_t j = offsets[i]; j < offsets[i + 1]; ++j) {
      int32_t t = tokens[j];
      if (t < 0 || t >= vocab || t == sep || t == stop) return ORC_ERR_CATALOG;
    }
  }

  int64_t total = offsets[K];
  int32_t capn = (int32_t)(total + 1);
  bnode* nodes = (bnode*)calloc((size_t)capn, sizeof(bnode));
  int32_t nb = 1;
  nodes[0].entry = -1;
  int32_t max_depth = 0;
  int rc = ORC_OK;
  for (int32_t i = 0; i < K && rc == ORC_OK; ++i) {
    int32_t cur = 0;
    int32_t len = (int32_t)(offsets[i + 1] - offsets[i]);
    if (len > max_depth) max_depth = len;
    for (int64_t j = offsets[i]; j < offsets[i + 1]; ++j) {
      int32_t nxt = bnode_find(&nodes[cur], tokens[j]);
      if (nxt < 0) {
        nxt = nb++;
        nodes[nxt].entry = -1;
        bnode_add(&nodes[cur], tokens[j], nxt);
      }
      cur = nxt;
    }
    if (nodes[cur].entry >= 0) rc = ORC_ERR_CATALOG; /* duplicate entry */
    else nodes[cur].entry = i;
  }
  if (rc != ORC_OK) {
    for (int32_t b = 0; b < nb; ++b) { free(nodes[b].ctok); free(nodes[b].cnode); }
    free(nodes);
    return rc;
  }

  int32_t* below = (int32_t*)malloc(sizeof(int32_t) * nb);
  count_terminals(nodes, nb, below);

  /* breadth-first numbering */
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * nb); /* bfs id -> build id */
  int32_t* bfs_of = (int32_t*)malloc(sizeof(int32_t) * nb); /* build id -> bfs id */
  int32_t head = 0, tail = 0;
  order[tail++] = 0;
  while (head < tail) {
    int32_t b = order[head++];
    bnode_sort(&nodes[b]);
    for (int32_t i = 0; i < nodes[b].nchild; ++i) order[tail++] = nodes[b].cnode[i];
  }
  for (int32_t i = 0; i < nb; ++i) bfs_of[order[i]] = i;

  orc_trie* t = (orc_trie*)calloc(1, sizeof(orc_trie));
  t->n_nodes = nb;
  t->n_entries = K;
  t->sep = sep;
  t->stop = stop;
  t->vocab = vocab;
  t->max_depth = max_depth;
  int32_t n_edges = 0;
  for (int32_t b = 0; b < nb; ++b) n_edges += nodes[b].nchild + (nodes[b].entry >= 0 ? 2 : 0);
  t->n_edges = n_edges;
  t->begin = (int32_t*)malloc(sizeof(int32_t) * (nb + 1));
  t->entry = (int32_t*)malloc(sizeof(int32_t) * nb);
  t->tok = (int32_t*)malloc(sizeof(int32_t) * (n_edges ? n_edges : 1));
  t->child = (int32_t*)malloc(sizeof(int32_t) * (n_edges ? n_edges : 1));
  t->live0 = (int32_t*)malloc(sizeof(int32_t) * (n_edges ? n_edges : 1));

  int32_t e = 0, cap = 0;
  for (int32_t id = 0; id < nb; ++id) {
    const bnode* n = &nodes[order[id]];
    t->begin[id] = e;
    t->entry[id] = n->entry;
    /* merge the sorted content edges with the (sorted) control edges */
    int32_t ctl_tok[2], ctl_child[2], nctl = 0;
    if (n->entry >= 0) {
      if (sep < stop) {
        ctl_tok[0] = sep; ctl_child[0] = CHILD_SEP; ctl_tok[1] = stop; ctl_child[1] = CHILD_STOP;
      } else {
        ctl_tok[0] = stop; ctl_child[0] = CHILD_STOP; ctl_tok[1] = sep; ctl_child[1] = CHILD_SEP;
      }
      nctl = 2;
    }
    int32_t i = 0, c = 0;
    while (i < n->nchild || c < nctl) {
      if (c >= nctl || (i < n->nchild && n->ctok[i] < ctl_tok[c])) {
        t->tok[e] = n->ctok[i];
        t->child[e] = bfs_of[n->cnode[i]];
        t->live0[e] = below[n->cnode[i]];
        ++i;
      } else {
        t->tok[e] = ctl_tok[c];
        t->child[e] = ctl_child[c];
        t->live0[e] = 0;
        ++c;
      }
      ++e;
    }
    if (e - t->begin[id] > cap) cap = e - t->begin[id];
  }
  t->begin[nb] = e;
  t->cap = cap;

  for (int32_t b = 0; b < nb; ++b) { free(nodes[b].ctok); free(nodes[b].cnode); }
  free(nodes); free(below); free(order); free(bfs_of);
  *out = t;
  return ORC_OK;
}

/* info: n_nodes, n_edges, n_entries, cap, max_depth, sep, stop, vocab */
void orc_trie_info(const orc_trie* t, int32_t* info) {
  info[0] = t->n_nodes; info[1] = t->n_edges; info[2] = t->n_entries; info[3] = t->cap;
  info[4] = t->max_depth; info[5] = t->sep; info[6] = t->stop; info[7] = t->vocab;
}

void orc_trie_csr(const orc_trie* t, int32_t* begin, int32_t* entry, int32_t* tok,
                  int32_t* child, int32_t* live0) {
  memcpy(begin, t->begin, sizeof(int32_t) * (t->n_nodes + 1));
  memcpy(entry, t->entry, sizeof(int32_t) * t->n_nodes);
  memcpy(tok, t->tok, sizeof(int32_t) * t->n_edges);
  memcpy(child, t->child, sizeof(int32_t) * t->n_edges);
  memcpy(live0, t->live0, sizeof(int32_t) * t->n_edges);
}

/* ------------------------------------------------------------------------- */
/* Decode state of one sequence                                               */
/* ------------------------------------------------------------------------- */

typedef struct {
  const orc_trie* t;
  int32_t k;
  int32_t node, depth, done, finished, status, n_emitted;
  int32_t* path;     /* [max_depth] content edges from the root */
  int32_t* live;     /* [n_edges] */
  unsigned char* spent; /* [n_entries] */
  int32_t* entries;  /* [k] catalog indices of completed pointers */
} orc_state;

orc_state* orc_state_new(const orc_trie* t, int32_t k) {
  orc_state* s = (orc_state*)calloc(1, sizeof(orc_state));
  s->t = t;
  s->k = k;
  s->path = (int32_t*)calloc((size_t)t->max_depth + 1, sizeof(int32_t));
  s->live = (int32_t*)malloc(sizeof(int32_t) * (t->n_edges ? t->n_edges : 1));
  memcpy(s->live, t->live0, sizeof(int32_t) * t->n_edges);
  s->spent = (unsigned char*)calloc((size_t)t->n_entries, 1);
  s->entries = (int32_t*)malloc(sizeof(int32_t) * (k > 0 ? k : 1));
  for (int32_t i = 0; i < k; ++i) s->entries[i] = -1;
  return s;
}

void orc_state_free(orc_state* s) {
  if (!s) return;
  free(s->path); free(s->live); free(s->spent); free(s->entries); free(s);
}

/* is edge e of the current node legal for this sequence? */
static int edge_legal(const orc_state* s, int32_t e) {
  const orc_trie* t = s->t;
  int32_t c = t->child[e];
  if (c >= 0) return s->live[e] > 0;
  int32_t ent = t->entry[s->node];
  if (ent < 0) return 0;
  if (s->spent[ent] && g_mutant != MUT_NO_SPENT_FLAG) return 0;
  int more = s->done + 1 < s->k;
  if (g_mutant == MUT_SEP_STOP_SWAPPED) more = !more;
  return c == CHILD_SEP ? more : !more;
}

/* legal tokens (and their edges) at the current node, ascending token order;
 * returns the count, or -1 when the sequence is finished or in error */
int32_t orc_state_legal(const orc_state* s, int32_t* toks, int32_t* edges) {
  if (s->finished || s->status != ORC_OK) return -1;
  const orc_trie* t = s->t;
  int32_t n = 0;
  for (int32_t e = t->begin[s->node]; e < t->begin[s->node + 1]; ++e) {
    if (edge_legal(s, e)) {
      if (toks) toks[n] = t->tok[e];
      if (edges) edges[n] = e;
      ++n;
    }
  }
  return n;
}

/* take token `tok` at the current node; returns the sequence status */
int32_t orc_state_advance(orc_state* s, int32_t tok) {
  if (s->finished || s->status != ORC_OK) return s->status != ORC_OK ? s->status : ORC_ERR_INVALID_ARG;
  const orc_trie* t = s->t;
  int32_t e = -1;
  for (int32_t i = t->begin[s->node]; i < t->begin[s->node + 1]; ++i)
    if (t->tok[i] == tok) { e = i; break; }
  if (e < 0 || !edge_legal(s, e)) {
    s->status = ORC_ERR_NOT_WALKABLE;
    return s->status;
  }
  s->n_emitted++;
  int32_t c = t->child[e];
  if (c >= 0) {
    s->path[s->depth++] = e;
    s->node = c;
    return ORC_OK;
  }
  /* a pointer completes: spend its terminal, release its path */
  int32_t ent = t->entry[s->node];
  s->spent[ent] = 1;
  if (g_mutant != MUT_NO_LIVE_DECREMENT)
    for (int32_t i = 0; i < s->depth; ++i) s->live[s->path[i]] -= 1;
  s->depth = 0;
  s->entries[s->done] = ent;
  s->done++;
  if (c == CHILD_SEP) s->node = 0;
  else s->finished = 1;
  return ORC_OK;
}

/* node, depth, done, finished, status, n_emitted */
void orc_state_info(const orc_state* s, int32_t* info) {
  info[0] = s->node; info[1] = s->depth; info[2] = s->done;
  info[3] = s->finished; info[4] = s->status; info[5] = s->n_emitted;
}

void orc_state_live(const orc_state* s, int32_t* live) {
  memcpy(live, s->live, sizeof(int32_t) * s->t->n_edges);
}

void orc_state_entries(const orc_state* s, int32_t* entries) {
  memcpy(entries, s->entries, sizeof(int32_t) * s->k);
}

/* ------------------------------------------------------------------------- */
/* Logits                                                                      */
/* ------------------------------------------------------------------------- */

/* element i of a row stored as fp32 (dtype 0) or as bf16 bit patterns (1),
 * widened exactly to double */
static double elem(const void* base, int dtype, int64_t i) {
  if (dtype == 0) return (double)((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* logit of token v: sum over i of h[i] * E[v][i] in index order, in fp64.
 * Every product is exact in fp64 (bf16 and fp32 significands are 8 and 24
 * bits).  *sumabs receives sum |h[i] E[v][i]| for error bounds. */
double orc_logit(const void* emb, int dtype, int32_t H, int32_t v, const void* h, double* sumabs) {
  int64_t row = (int64_t)(g_mutant == MUT_ROW_OFF_BY_ONE ? v + 1 : v) * H;
  int32_t n = g_mutant == MUT_DROP_LAST_TERM ? H - 1 : H;
  double acc = 0.0, a = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    double p = elem(h, dtype, i) * elem(emb, dtype, row + i);
    acc += p;
    a += fabs(p);
  }
  if (sumabs) *sumabs = a;
  return acc;
}

/* all V logits of one hidden vector (the dense head) */
void orc_dense_logits(const void* emb, int dtype, int32_t V, int32_t H, const void* h, double* out) {
  for (int32_t v = 0; v < V; ++v) {
    int32_t vv = (g_mutant == MUT_ROW_OFF_BY_ONE && v == V - 1) ? V - 2 : v; /* keep in range */
    out[v] = orc_logit(emb, dtype, H, vv, h, NULL);
  }
}

/* ------------------------------------------------------------------------- */
/* Greedy decode                                                               */
/* ------------------------------------------------------------------------- */

/* One greedy pick: legal set, logits, first maximum in ascending token order
 * (ties to the lower id).  Records the winner's logit, the top-two margin
 * (+inf with one candidate), the larger sum|p| of the top two, and the size of
 * the legal set.  Returns the token (the state is not advanced), or -1 when the
 * sequence is inactive or its mask is empty (then EMPTY_MASK is set). */
static int32_t greedy_step(orc_state* s, const void* emb, int dtype, int32_t H, const void* h,
                           int32_t* scratch_tok, double* best_out, double* margin_out,
                           double* sumabs_out, int32_t* nlegal_out) {
  int32_t n = orc_state_legal(s, scratch_tok, NULL);
  if (nlegal_out) *nlegal_out = n < 0 ? 0 : n;
  if (n < 0) return -1;
  if (n == 0) {
    s->status = ORC_ERR_EMPTY_MASK;
    return -1;
  }
  int32_t win = -1;
  double best = 0.0, second = -INFINITY, best_abs = 0.0, second_abs = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    double a;
    double l = orc_logit(emb, dtype, H, scratch_tok[j], h, &a);
    int better = (win < 0) || (g_mutant == MUT_TIE_HIGHER_ID ? l >= best : l > best);
    if (better) {
      if (win >= 0) { second = best; second_abs = best_abs; }
      win = scratch_tok[j];
      best = l;
      best_abs = a;
    } else if (l > second || (l == second && second_abs < a)) {
      second = l;
      second_abs = a;
    }
  }
  if (best_out) *best_out = best;
  if (margin_out) *margin_out = g_mutant == MUT_MARGIN_ZERO ? 0.0 : n > 1 ? best - second : INFINITY;
  if (sumabs_out)
    *sumabs_out = g_mutant != MUT_SUMABS_WINNER && n > 1 && second_abs > best_abs ? second_abs : best_abs;
  return win;
}

/* Greedy decode of B independent sequences over T steps.
 * hidden: [T][B][H] (fp32 or bf16 bits, same dtype as emb).
 * follow: NULL for the plain greedy decode, or [B][T] tokens to advance by
 * (teacher forcing, "Understanding Inference for Systems Engineers", Part 8
 * "Correctness"): at each step the oracle still records its own greedy pick
 * and its statistics from the current state, then advances by follow[b][t]
 * when that is >= 0 (a token that is not legal sets NOT_WALKABLE) and by its
 * own pick otherwise.
 * Outputs (any may be NULL): tokens [B][T] (the oracle's pick, -1 padded),
 * len [B], entries [B][k], status [B] (NOT_DONE when no stop was emitted
 * within T steps), and per step best logit, top-two margin, sum|p| and
 * legal-set size, each [B][T].
 * Sequences are decoded one after another; nothing is shared between them. */
int orc_decode(const orc_trie* t, int32_t k, const void* emb, int dtype, int32_t V, int32_t H,
               const void* hidden, int32_t B, int32_t T, const int32_t* follow, int32_t* tokens,
               int32_t* len, int32_t* entries, int32_t* status, double* best, double* margin,
               double* sumabs, int32_t* nlegal) {
  if (k < 1 || k > t->n_entries) return ORC_ERR_K;
  if (V != t->vocab || H < 1 || B < 1 || T < 0) return ORC_ERR_INVALID_ARG;
  size_t esz = dtype == 0 ? 4 : 2;
  int32_t* scratch = (int32_t*)malloc(sizeof(int32_t) * (t->cap ? t->cap : 1));
  for (int32_t b = 0; b < B; ++b) {
    orc_state* s = orc_state_new(t, k);
    for (int32_t step = 0; step < T; ++step) {
      const void* h = (const char*)hidden + ((size_t)step * B + b) * (size_t)H * esz;
      int64_t o = (int64_t)b * T + step;
      int32_t tok = greedy_step(s, emb, dtype, H, h, scratch, best ? &best[o] : NULL,
                                margin ? &margin[o] : NULL, sumabs ? &sumabs[o] : NULL,
                                nlegal ? &nlegal[o] : NULL);
      if (tokens) tokens[o] = tok;
      if (tok < 0) {
        if (best) best[o] = NAN;
        if (margin) margin[o] = NAN;
        if (sumabs) sumabs[o] = NAN;
        continue;
      }
      int32_t take = tok;
      if (follow && follow[o] >= 0 && g_mutant != MUT_FOLLOW_IGNORED) take = follow[o];
      orc_state_advance(s, take);
    }
    if (s->status == ORC_OK && !s->finished) s->status = ORC_ERR_NOT_DONE;
    if (len) len[b] = s->n_emitted;
    if (entries) memcpy(&entries[(int64_t)b * k], s->entries, sizeof(int32_t) * k);
    if (status) status[b] = s->status;
    orc_state_free(s);
  }
  free(scratch);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Character-level catalogs                                                    */
/* ------------------------------------------------------------------------- */

/* Source: the review of arXiv 2608.12574 (fields pith_extraction.key_machinery
 * and core_discovery).  The catalog is a set C of byte strings and the
 * vocabulary maps each token id v to a byte string b(v); an answer is one
 * string of C spelled by a sequence of tokens, then the stop token.  By the
 * next-token mask definition (page "GLRMask", with b as the token-to-bytes
 * map) the legal set after tokens u is
 *     Mask(u) = { v : some tokens w make b(u v w) a string of C, v != stop }
 *               plus stop when b(u) is itself a string of C.
 * When every byte that occurs in C is also a token of its own (byte-level
 * vocabularies), every remainder of a string can be spelled, so a content
 * token v is legal exactly when b(u) b(v) is a prefix of some string of C.
 * This section computes that set by enumeration: for each catalog string that
 * starts with b(u), every token spelling the next 1, 2, ... bytes of it.  The
 * page's trie, Aho-Corasick matcher and precomputed valid[node] sets are the
 * fast way to the same sets; nothing of them is used here.  Readings: empty
 * byte strings are control or unused tokens and never content; the sep and
 * stop ids are never content; duplicate strings are rejected.  One string is
 * chosen (k = 1): sep is never legal. */

typedef struct {
  int32_t K, V, sep, stop, max_len, max_tok;
  uint8_t* bytes;  /* catalog strings, back to back */
  int64_t* off;    /* [K+1] */
  int32_t* order;  /* catalog indices in lexicographic byte order */
  uint8_t* tb;     /* token byte strings, back to back */
  int64_t* toff;   /* [V+1] */
  int32_t* torder; /* content token ids ordered by (bytes, id) */
  int32_t nt;      /* number of content tokens */
} orc_cs;

static const orc_cs* g_cs_sort; /* context of the two qsort comparators below */

static int cmp_bytes(const uint8_t* a, int64_t la, const uint8_t* b, int64_t lb) {
  int64_t n = la < lb ? la : lb;
  int c = n ? memcmp(a, b, (size_t)n) : 0;
  if (c) return c;
  return la < lb ? -1 : la > lb ? 1 : 0;
}

static int cmp_str_idx(const void* x, const void* y) {
  int32_t i = *(const int32_t*)x, j = *(const int32_t*)y;
  const orc_cs* c = g_cs_sort;
  return cmp_bytes(c->bytes + c->off[i], c->off[i + 1] - c->off[i], c->bytes + c->off[j], c->off[j + 1] - c->off[j]);
}

static int cmp_tok_idx(const void* x, const void* y) {
  int32_t i = *(const int32_t*)x, j = *(const int32_t*)y;
  const orc_cs* c = g_cs_sort;
  int r = cmp_bytes(c->tb + c->toff[i], c->toff[i + 1] - c->toff[i], c->tb + c->toff[j], c->toff[j + 1] - c->toff[j]);
  return r ? r : (i < j ? -1 : i > j ? 1 : 0);
}

void orc_cs_free(orc_cs* c) {
  if (!c) return;
  free(c->bytes); free(c->off); free(c->order); free(c->tb); free(c->toff); free(c->torder);
  free(c);
}

/* Validates and copies a character catalog.  Errors: INVALID_ARG for sizes
 * and control ids, CATALOG for an empty or duplicate string or a byte of a
 * string that no single-byte content token spells. */
int orc_cs_build(const uint8_t* bytes, const int64_t* off, int32_t K, const uint8_t* tbytes,
                 const int64_t* toff, int32_t V, int32_t sep, int32_t stop, orc_cs** out) {
  *out = NULL;
  if (K < 1 || V < 2 || sep < 0 || sep >= V || stop < 0 || stop >= V || sep == stop) return ORC_ERR_INVALID_ARG;
  if (off[0] != 0 || toff[0] != 0) return ORC_ERR_INVALID_ARG;
  orc_cs* c = (orc_cs*)calloc(1, sizeof(orc_cs));
  c->K = K; c->V = V; c->sep = sep; c->stop = stop;
  c->off = (int64_t*)malloc(sizeof(int64_t) * (K + 1));
  memcpy(c->off, off, sizeof(int64_t) * (K + 1));
  c->bytes = (uint8_t*)malloc((size_t)off[K] + 1);
  memcpy(c->bytes, bytes, (size_t)off[K]);
  c->toff = (int64_t*)malloc(sizeof(int64_t) * (V + 1));
  memcpy(c->toff, toff, sizeof(int64_t) * (V + 1));
  c->tb = (uint8_t*)malloc((size_t)toff[V] + 1);
  memcpy(c->tb, tbytes, (size_t)toff[V]);
  int single[256] = {0};
  c->torder = (int32_t*)malloc(sizeof(int32_t) * V);
  for (int32_t v = 0; v < V; ++v) {
    int64_t L = toff[v + 1] - toff[v];
    if (L < 0) { orc_cs_free(c); return ORC_ERR_INVALID_ARG; }
    if (L == 0 || v == sep || v == stop) continue;
    c->torder[c->nt++] = v;
    if (L > c->max_tok) c->max_tok = (int32_t)L;
    if (L == 1) single[tbytes[toff[v]]] = 1;
  }
  c->order = (int32_t*)malloc(sizeof(int32_t) * K);
  for (int32_t i = 0; i < K; ++i) {
    int64_t L = off[i + 1] - off[i];
    if (L <= 0) { orc_cs_free(c); return ORC_ERR_CATALOG; }
    if (L > c->max_len) c->max_len = (int32_t)L;
    for (int64_t j = off[i]; j < off[i + 1]; ++j)
      if (!single[bytes[j]]) { orc_cs_free(c); return ORC_ERR_CATALOG; }
    c->order[i] = i;
  }
  g_cs_sort = c;
  qsort(c->order, (size_t)K, sizeof(int32_t), cmp_str_idx);
  qsort(c->torder, (size_t)c->nt, sizeof(int32_t), cmp_tok_idx);
  for (int32_t i = 1; i < K; ++i)
    if (cmp_str_idx(&c->order[i - 1], &c->order[i]) == 0) { orc_cs_free(c); return ORC_ERR_CATALOG; }
  *out = c;
  return ORC_OK;
}

/* max_len, max_tok, number of content tokens */
void orc_cs_info(const orc_cs* c, int32_t* info) {
  info[0] = c->max_len; info[1] = c->max_tok; info[2] = c->nt;
}

/* first position in the sorted catalog whose string is >= p (bytes) */
static int32_t cs_lower(const orc_cs* c, const uint8_t* p, int64_t n) {
  int32_t lo = 0, hi = c->K;
  while (lo < hi) {
    int32_t mid = (lo + hi) / 2, i = c->order[mid];
    if (cmp_bytes(c->bytes + c->off[i], c->off[i + 1] - c->off[i], p, n) < 0) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

/* first position in the sorted content tokens whose bytes are >= p */
static int32_t tok_lower(const orc_cs* c, const uint8_t* p, int64_t n) {
  int32_t lo = 0, hi = c->nt;
  while (lo < hi) {
    int32_t mid = (lo + hi) / 2, v = c->torder[mid];
    if (cmp_bytes(c->tb + c->toff[v], c->toff[v + 1] - c->toff[v], p, n) < 0) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

/* The legal set after the emitted bytes p[0..n): token ids in ascending
 * order into out (room for V), stop included when p is a catalog string.
 * Returns the count (0: empty mask).  mark: scratch of V bytes, zeroed. */
static int32_t cs_mask(const orc_cs* c, const uint8_t* p, int64_t n, int32_t* out, uint8_t* mark) {
  int32_t any = 0, stop_ok = 0;
  for (int32_t pos = cs_lower(c, p, n); pos < c->K; ++pos) {
    const int32_t i = c->order[pos];
    const uint8_t* s = c->bytes + c->off[i];
    const int64_t L = c->off[i + 1] - c->off[i];
    if (L < n || (n && memcmp(s, p, (size_t)n) != 0)) break; /* past the strings that start with p */
    if (L == n) {
      stop_ok = 1;
      continue;
    }
    if (g_mutant == MUT_CS_FIRST_BYTE) {
      for (int32_t q = 0; q < c->nt; ++q) {
        const int32_t v = c->torder[q];
        if (c->tb[c->toff[v]] == s[n] && !mark[v]) { mark[v] = 1; any = 1; }
      }
      continue;
    }
    /* every token spelling s[n .. n+l), l = 1 .. the bytes left */
    const int64_t top = L - n < c->max_tok ? L - n : c->max_tok;
    for (int64_t l = 1; l <= top; ++l) {
      for (int32_t q = tok_lower(c, s + n, l); q < c->nt; ++q) {
        const int32_t v = c->torder[q];
        if (c->toff[v + 1] - c->toff[v] != l || memcmp(c->tb + c->toff[v], s + n, (size_t)l) != 0) break;
        if (!mark[v]) { mark[v] = 1; any = 1; }
      }
    }
  }
  if (stop_ok && g_mutant == MUT_CS_STOP_LEAF_ONLY && any) stop_ok = 0;
  if (stop_ok) mark[c->stop] = 1;
  int32_t k = 0;
  for (int32_t v = 0; v < c->V; ++v)
    if (mark[v]) { out[k++] = v; mark[v] = 0; }
  return k;
}

/* Legal set after the byte prefix p[0..n) (ascending token ids into out,
 * room for V); returns the count. */
int32_t orc_cs_mask(const orc_cs* c, const uint8_t* p, int64_t n, int32_t* out) {
  uint8_t* mark = (uint8_t*)calloc((size_t)c->V, 1);
  int32_t k = cs_mask(c, p, n, out, mark);
  free(mark);
  return k;
}

/* Greedy decode of B sequences over a character catalog (k = 1), hidden
 * [T][B][H]: at each step the legal set above, one fp64 logit per legal
 * token (orc_logit), the first maximum in ascending id order, then the
 * token's bytes appended (stop: the string chosen, sequence done).  follow
 * ([B][T] or NULL): teacher forcing as in orc_decode.  Outputs as for
 * orc_decode, with entry [B] the catalog index of the chosen string (-1
 * when none) and status EMPTY_MASK, NOT_WALKABLE (a forced token outside the
 * legal set) or NOT_DONE (no stop within T steps). */
int orc_cs_decode(const orc_cs* c, const void* emb, int dtype, int32_t H, const void* hidden, int32_t B, int32_t T,
                  const int32_t* follow, int32_t* tokens, int32_t* len, int32_t* entry, int32_t* status,
                  double* best, double* margin, double* sumabs, int32_t* nlegal) {
  if (H < 1 || B < 1 || T < 0) return ORC_ERR_INVALID_ARG;
  const size_t esz = dtype == 0 ? 4 : 2;
  int32_t* legal = (int32_t*)malloc(sizeof(int32_t) * c->V);
  uint8_t* mark = (uint8_t*)calloc((size_t)c->V, 1);
  uint8_t* pre = (uint8_t*)malloc((size_t)c->max_len + 1);
  for (int32_t b = 0; b < B; ++b) {
    int64_t n = 0;
    int32_t st = ORC_OK, fin = 0, emitted = 0, ent = -1;
    for (int32_t t = 0; t < T; ++t) {
      const int64_t o = (int64_t)b * T + t;
      if (tokens) tokens[o] = -1;
      if (best) best[o] = NAN;
      if (margin) margin[o] = NAN;
      if (sumabs) sumabs[o] = NAN;
      if (nlegal) nlegal[o] = 0;
      if (fin || st != ORC_OK) continue;
      const int32_t k = cs_mask(c, pre, n, legal, mark);
      if (nlegal) nlegal[o] = k;
      if (k == 0) {
        st = ORC_ERR_EMPTY_MASK;
        continue;
      }
      const void* h = (const char*)hidden + ((size_t)t * B + b) * (size_t)H * esz;
      int32_t win = -1;
      double bl = 0.0, second = -INFINITY, ba = 0.0, sa2 = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        double a;
        const double l = orc_logit(emb, dtype, H, legal[j], h, &a);
        if (win < 0 || l > bl) {
          if (win >= 0) { second = bl; sa2 = ba; }
          win = legal[j]; bl = l; ba = a;
        } else if (l > second || (l == second && sa2 < a)) {
          second = l; sa2 = a;
        }
      }
      if (tokens) tokens[o] = win;
      if (best) best[o] = bl;
      if (margin) margin[o] = k > 1 ? bl - second : INFINITY;
      if (sumabs) sumabs[o] = k > 1 && sa2 > ba ? sa2 : ba;
      int32_t take = win;
      if (follow && follow[o] >= 0) {
        take = follow[o];
        int ok = 0;
        for (int32_t j = 0; j < k; ++j) ok |= legal[j] == take;
        if (!ok) {
          st = ORC_ERR_NOT_WALKABLE;
          continue;
        }
      }
      emitted++;
      if (take == c->stop) {
        fin = 1;
        const int32_t pos = cs_lower(c, pre, n);
        ent = c->order[pos]; /* the string equal to the prefix: legal stop guarantees it */
      } else {
        const int64_t tl = c->toff[take + 1] - c->toff[take];
        memcpy(pre + n, c->tb + c->toff[take], (size_t)tl);
        n += tl;
      }
    }
    if (st == ORC_OK && !fin) st = ORC_ERR_NOT_DONE;
    if (len) len[b] = emitted;
    if (entry) entry[b] = fin ? ent : -1;
    if (status) status[b] = st;
  }
  free(legal);
  free(mark);
  free(pre);
  return ORC_OK;
}
