/* Host-side validation of every libjetblock entry point, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer from a host-only compile of
 * the library (no device code) by tests/test_oracle_sanitized.py.
 *
 * Every call here is one the library must reject before it reaches the HIP
 * runtime: a bad shape field, one NULL or misaligned pointer, a missing or
 * short workspace.  The pointers are stand-in addresses that are never
 * dereferenced; a call that got past validation would reach HIP, which this
 * driver only allows when no GPU is visible (then HIP reports the failure).
 * Workspace-size queries run on shapes up to the documented limits so that an
 * integer overflow in the planning code shows up as a UBSan report. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/jetblock.h"

int hipGetDeviceCount(int* count);

static int fails = 0, checks = 0;
#define EXPECT(cond, ...) do { ++checks; if (!(cond)) { ++fails; fprintf(stderr, "line %d: ", __LINE__); \
  fprintf(stderr, __VA_ARGS__); fprintf(stderr, " [last error: %s]\n", jb_last_error()); } } while (0)

#define NP 40
static void* P[NP];
#define GOOD ((void*)(uintptr_t)0x100000)
#define WS_OK ((size_t)1 << 60)

/* pointer-argument kinds: R required (16-byte aligned), S required scalars (4-byte aligned),
 * O optional (16-byte aligned when set), C one of a group that is all set or all NULL,
 * W the workspace (256-byte aligned), N ignored */
typedef jb_status (*caller)(const jb_shape* s, size_t wsb);
typedef struct { const char* name; const char* kinds; caller call; int decode; int has_ws; } entry;

#define A(i) (P[i])
/* x q k v alpha beta W1 b1 W2 b2 S0 conv_in o S_final conv_out workspace */
#define K_PREFILL "RRRRSSROROOORROW"
/* q k v alpha beta wq wk wv S0 cache_{q,k,v}_in o S_final cache_{q,k,v}_out workspace */
#define K_STATIC "RRRSSRRROCCCRROOOW"
/* x q k v alpha beta W1 b1 W2 b2 S0 conv_in dout dS_final dconv_out dx dq dk dv dalpha dbeta
 * dW1 db1 dW2 db2 dS0 dconv_in workspace */
#define K_BACKWARD "RRRRSSROROOOROORRRRSSRSRSRRW"
static jb_status c_prefill(const jb_shape* s, size_t wsb) {
  return jb_prefill(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), A(11), A(12), A(13), A(14),
                    A(15), wsb, NULL);
}
static jb_status c_prefill_noalloc(const jb_shape* s, size_t wsb) {
  (void)wsb;
  return jb_prefill_noalloc(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), A(11), A(12), A(13),
                            A(14), NULL);
}
static jb_status c_decode_step(const jb_shape* s, size_t wsb) {
  return jb_decode_step(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), A(11), A(12), A(13),
                        A(14), A(15), wsb, NULL);
}
static int64_t g_total = 100;
static jb_status c_prefill_varlen(const jb_shape* s, size_t wsb) {
  return jb_prefill_varlen(s, g_total, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), A(11),
                           A(12), A(13), A(14), A(15), A(16), wsb, NULL);
}
static jb_status c_project(const jb_shape* s, size_t wsb) {
  return jb_project(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), A(11), A(12), A(13), A(14),
                    A(15), A(16), A(17), A(18), wsb, NULL);
}
static jb_status c_prefill_from_x(const jb_shape* s, size_t wsb) {
  return jb_prefill_from_x(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), A(11), A(12), A(13),
                           A(14), A(15), A(16), A(17), wsb, NULL);
}
static jb_status c_decode_step_from_x(const jb_shape* s, size_t wsb) {
  return jb_decode_step_from_x(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), A(11), A(12),
                               A(13), A(14), A(15), A(16), A(17), wsb, NULL);
}
static jb_status c_prefill_static(const jb_shape* s, size_t wsb) {
  return jb_prefill_static(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), A(11), A(12), A(13),
                           A(14), A(15), A(16), A(17), wsb, NULL);
}
static jb_status c_decode_step_static(const jb_shape* s, size_t wsb) {
  (void)wsb;
  return jb_decode_step_static(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), A(11), A(12),
                               A(13), A(14), A(15), A(16), NULL);
}
static jb_status c_backward(const jb_shape* s, size_t wsb) {
  return jb_backward(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), A(11), A(12), A(13), A(14),
                     A(15), A(16), A(17), A(18), A(19), A(20), A(21), A(22), A(23), A(24), A(25), A(26), A(27), wsb,
                     NULL);
}
static jb_status c_gen_taps(const jb_shape* s, size_t wsb) {
  (void)wsb;
  return jb_gen_taps(s, A(0), A(1), A(2), A(3), A(4), A(5), NULL);
}
static jb_status c_gen_conv(const jb_shape* s, size_t wsb) {
  (void)wsb;
  return jb_gen_conv(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), NULL);
}
static jb_status c_prologue(const jb_shape* s, size_t wsb) {
  (void)wsb;
  return jb_prologue(s, A(0), A(1), A(2), A(3), A(4), A(5), NULL);
}
static jb_status c_decode_update(const jb_shape* s, size_t wsb) {
  (void)wsb;
  return jb_decode_update(s, A(0), A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8), A(9), A(10), NULL);
}

static const entry entries[] = {
  {"jb_prefill", K_PREFILL, c_prefill, 0, 1},
  {"jb_prefill_noalloc", "RRRRSSROROOORRO", c_prefill_noalloc, 0, 0},
  {"jb_decode_step", "RRRRRRRRSSRORORN", c_decode_step, 1, 0},
  {"jb_prefill_varlen", "SRRRRSSROROOORROW", c_prefill_varlen, 0, 1},
  {"jb_project", "RRRRRORORORORRRSSRN", c_project, 0, 0},
  {"jb_prefill_from_x", "RRRRRORORORO" "OORROW", c_prefill_from_x, 0, 1},
  {"jb_decode_step_from_x", "RRRRRRRRRORORORORW", c_decode_step_from_x, 1, 1},
  {"jb_prefill_static", K_STATIC, c_prefill_static, 0, 1},
  {"jb_decode_step_static", "RRRRRRRRRRRSSRRRR", c_decode_step_static, 1, 0},
  {"jb_backward", K_BACKWARD, c_backward, 0, 1},
  {"jb_gen_taps", "RROROR", c_gen_taps, 0, 0},
  {"jb_gen_conv", "RRORORORR", c_gen_conv, 0, 0},
  {"jb_prologue", "RRSRRR", c_prologue, 0, 0},
  {"jb_decode_update", "RRRRRRRSSRR", c_decode_update, 1, 0},
};

static jb_shape base_shape(int decode) {
  jb_shape s = {2, decode ? 1 : 130, 4, 64, 128, 256, 32, 4, 0, JB_BF16, JB_BF16, 0};
  return s;
}

static void reset_ptrs(const char* kinds) {
  for (int i = 0; i < NP; ++i) P[i] = NULL;
  for (int i = 0; kinds[i]; ++i) P[i] = kinds[i] == 'N' ? NULL : GOOD;
}

static void check_entry(const entry* e) {
  const int n = (int)strlen(e->kinds);
  jb_shape s = base_shape(e->decode);
  /* jb_prefill_static needs segments for a nonzero workspace */
  if (!strcmp(e->name, "jb_prefill_static")) s.flags = JB_FLAG_SEGMENT(1);
  /* jb_prefill_noalloc: a shape whose workspace exceeds the file-scope scratch */
  jb_shape big = s;
  big.B = 64; big.T = 65536; big.H = 32;

  /* shape fields */
  const struct { const char* what; int field; int value; jb_status want; } bad[] = {
    {"B", 0, 0, JB_ERR_INVALID_ARG}, {"B", 0, 65536, JB_ERR_UNSUPPORTED}, {"H", 2, 0, JB_ERR_UNSUPPORTED},
    {"H", 2, 33, JB_ERR_UNSUPPORTED}, {"dk", 3, 48, JB_ERR_UNSUPPORTED}, {"dv", 4, 32, JB_ERR_UNSUPPORTED},
    {"d_model", 5, 100, JB_ERR_UNSUPPORTED}, {"d_model", 5, 0, JB_ERR_UNSUPPORTED},
    {"gen_hidden", 6, 16, JB_ERR_UNSUPPORTED}, {"taps", 7, 3, JB_ERR_UNSUPPORTED},
    {"chunk", 8, 32, JB_ERR_UNSUPPORTED}, {"io_dtype", 9, 7, JB_ERR_INVALID_ARG},
    {"out_dtype", 10, -1, JB_ERR_INVALID_ARG}, {"flags", 11, 1, JB_ERR_INVALID_ARG},
  };
  for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
    jb_shape t = s;
    ((int32_t*)&t)[bad[i].field] = bad[i].value;
    reset_ptrs(e->kinds);
    jb_status st = e->call(&t, WS_OK);
    EXPECT(st == bad[i].want, "%s: %s = %d gave %s", e->name, bad[i].what, bad[i].value, jb_status_string(st));
    EXPECT(strstr(jb_last_error(), e->name) && strstr(jb_last_error(), bad[i].what), "%s: message for %s", e->name,
           bad[i].what);
  }
  {
    jb_shape t = s;
    t.T = e->decode ? 2 : -1;
    reset_ptrs(e->kinds);
    jb_status st = e->call(&t, WS_OK);
    EXPECT(st == JB_ERR_INVALID_ARG, "%s: T = %d gave %s", e->name, t.T, jb_status_string(st));
    reset_ptrs(e->kinds);
    st = e->call(NULL, WS_OK);
    EXPECT(st == JB_ERR_INVALID_ARG, "%s: NULL shape gave %s", e->name, jb_status_string(st));
    if (!e->decode) {
      t = s;
      t.B = 65535; t.T = 1 << 20; t.H = 32;  /* tensors beyond the supported 2^40 elements */
      reset_ptrs(e->kinds);
      st = e->call(&t, WS_OK);
      EXPECT(st == JB_ERR_UNSUPPORTED, "%s: oversize shape gave %s", e->name, jb_status_string(st));
    }
  }

  /* one pointer at a time: NULL, then misaligned */
  for (int i = 0; i < n; ++i) {
    const char k = e->kinds[i];
    if (k == 'N') continue;
    /* calls that would pass validation are kept from HIP by a short workspace; entry points
     * without a workspace only get calls that must fail */
    const jb_shape* sh = !strcmp(e->name, "jb_prefill_noalloc") ? &big : &s;
    if (k == 'R' || k == 'S' || k == 'C') {
      reset_ptrs(e->kinds);
      P[i] = NULL;
      jb_status st = e->call(sh, e->has_ws ? 0 : WS_OK);
      EXPECT(st == JB_ERR_INVALID_ARG, "%s: NULL pointer argument %d gave %s", e->name, i, jb_status_string(st));
    }
    if (k == 'O' && (e->has_ws || !strcmp(e->name, "jb_prefill_noalloc"))) {
      reset_ptrs(e->kinds);
      P[i] = NULL;  /* accepted: the call then stops at the workspace */
      jb_status st = e->call(sh, 0);
      EXPECT(st == JB_ERR_WORKSPACE, "%s: NULL optional argument %d gave %s", e->name, i, jb_status_string(st));
    }
    if (k != 'W') {
      reset_ptrs(e->kinds);
      P[i] = (char*)GOOD + (k == 'S' ? 2 : 8);
      jb_status st = e->call(sh, e->has_ws ? 0 : WS_OK);
      EXPECT(st == JB_ERR_INVALID_ARG, "%s: misaligned pointer argument %d gave %s", e->name, i,
             jb_status_string(st));
      EXPECT(strstr(jb_last_error(), "aligned") != NULL, "%s: message for misaligned argument %d", e->name, i);
    }
  }

  /* the workspace: missing, short, misaligned */
  if (e->has_ws) {
    int w = (int)(strchr(e->kinds, 'W') - e->kinds);
    reset_ptrs(e->kinds);
    P[w] = NULL;
    jb_status st = e->call(&s, WS_OK);
    EXPECT(st == JB_ERR_WORKSPACE, "%s: NULL workspace gave %s", e->name, jb_status_string(st));
    reset_ptrs(e->kinds);
    st = e->call(&s, 0);
    EXPECT(st == JB_ERR_WORKSPACE, "%s: short workspace gave %s", e->name, jb_status_string(st));
    reset_ptrs(e->kinds);
    P[w] = (char*)GOOD + 128;
    st = e->call(&s, WS_OK);
    EXPECT(st == JB_ERR_INVALID_ARG, "%s: misaligned workspace gave %s", e->name, jb_status_string(st));
  }
}

/* workspace queries over shapes up to the documented limits */
static void check_sizes(void) {
  const int dks[] = {32, 64, 96, 128}, dvs[] = {64, 128, 256};
  const int64_t Ts[] = {0, 1, 63, 64, 65, 4096, 65536, 262144, 1 << 24, 1 << 30, (1 << 30) + 1, 0x7fffffff};
  const int Bs[] = {1, 2, 255, 256, 65535}, Hs[] = {1, 8, 32};
  for (size_t a = 0; a < 4; ++a)
    for (size_t b = 0; b < 3; ++b)
      for (size_t t = 0; t < sizeof(Ts) / sizeof(Ts[0]); ++t)
        for (size_t bi = 0; bi < sizeof(Bs) / sizeof(Bs[0]); ++bi)
          for (size_t hi = 0; hi < 3; ++hi)
            for (int seg = 0; seg <= 65535; seg += 65535) {
              jb_shape s = {Bs[bi], (int32_t)Ts[t], Hs[hi], dks[a], dvs[b], 2048, 32, 4, 64, JB_BF16, JB_F32,
                            seg ? JB_FLAG_SEGMENT(seg) : 0};
              const int64_t tok = (int64_t)s.B * s.T;
              const int ok = tok * s.H * 2048 < ((int64_t)1 << 40) && s.T <= (1 << 30);
              size_t bytes = 0;
              jb_status st = jb_prefill_workspace_size(&s, &bytes);
              EXPECT(ok ? st == JB_OK : st == JB_ERR_UNSUPPORTED, "prefill size B=%d T=%d H=%d: %s", s.B, s.T, s.H,
                     jb_status_string(st));
              if (st == JB_OK)
                EXPECT(bytes >= (size_t)tok * s.H * 16, "prefill workspace %zu below the taps", bytes);
              st = jb_prefill_varlen_workspace_size(&s, tok / 2, &bytes);
              EXPECT(ok ? st == JB_OK || tok / 2 > 0x7fffffff : st != JB_OK, "varlen size: %s", jb_status_string(st));
              st = jb_prefill_static_workspace_size(&s, &bytes);
              st = jb_project_workspace_size(&s, &bytes);
              EXPECT(ok ? st == JB_OK : st != JB_OK, "project size: %s", jb_status_string(st));
              st = jb_prefill_from_x_workspace_size(&s, &bytes);
              EXPECT(ok ? st == JB_OK : st != JB_OK, "prefill_from_x size: %s", jb_status_string(st));
              if (!seg) {
                st = jb_backward_workspace_size(&s, &bytes);
                (void)st;
              }
              s.T = 1; s.flags = 0;
              st = jb_decode_workspace_size(&s, &bytes);
              EXPECT(st == JB_OK && bytes == 0, "decode size: %s", jb_status_string(st));
              st = jb_decode_step_from_x_workspace_size(&s, &bytes);
              EXPECT(st == JB_OK, "decode_step_from_x size: %s", jb_status_string(st));
            }
  jb_shape s = base_shape(0);
  EXPECT(jb_prefill_workspace_size(&s, NULL) == JB_ERR_INVALID_ARG, "NULL bytes");
  size_t bytes;
  EXPECT(jb_prefill_varlen_workspace_size(&s, -1, &bytes) == JB_ERR_INVALID_ARG, "negative total_tokens");
  EXPECT(jb_prefill_varlen_workspace_size(&s, (int64_t)s.B * s.T + 1, &bytes) == JB_ERR_INVALID_ARG,
         "total_tokens above B*T");
  s.io_dtype = JB_F32;
  EXPECT(jb_project_workspace_size(&s, &bytes) == JB_ERR_UNSUPPORTED, "fp32 projections");
  EXPECT(jb_backward_workspace_size(&s, &bytes) == JB_ERR_UNSUPPORTED, "fp32 backward");
  s.dk = 128; s.dv = 256;
  EXPECT(jb_prefill_workspace_size(&s, &bytes) == JB_OK, "fp32 size query");
  reset_ptrs(K_PREFILL);
  EXPECT(c_prefill(&s, WS_OK) == JB_ERR_UNSUPPORTED, "fp32 prefill above 64x64 tiles");
}

static void check_misc(void) {
  EXPECT(jb_last_error()[0] == 0, "last error starts empty");
  EXPECT(!strcmp(jb_status_string(JB_OK), "JB_OK"), "status string");
  EXPECT(!strcmp(jb_status_string((jb_status)99), "JB_ERR_UNKNOWN"), "unknown status string");
  EXPECT(jb_version() >= 10000, "version");
  float* f = (float*)GOOD;
  EXPECT(jb_probe_mfma(3, f, f, f, NULL) == JB_ERR_INVALID_ARG, "probe kind");
  EXPECT(jb_probe_mfma(0, NULL, f, f, NULL) == JB_ERR_INVALID_ARG, "probe NULL");
  /* the static-conv caches are all or none */
  jb_shape s = base_shape(0);
  s.flags = JB_FLAG_SEGMENT(1);
  reset_ptrs(K_STATIC);
  P[9] = P[10] = P[11] = NULL;
  EXPECT(c_prefill_static(&s, 0) == JB_ERR_WORKSPACE, "static prefill without caches");
  P[10] = GOOD;
  EXPECT(c_prefill_static(&s, 0) == JB_ERR_INVALID_ARG, "static prefill with one cache");
  /* the backward takes no segment flag */
  s = base_shape(0);
  s.flags = JB_FLAG_SEGMENT(2);
  reset_ptrs(K_BACKWARD);
  EXPECT(c_backward(&s, WS_OK) == JB_ERR_INVALID_ARG, "backward with flags");
}

int main(void) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == 0 && ndev > 0) {
    printf("skipped: a GPU is visible and this driver passes stand-in pointers\n");
    return 0;
  }
  check_misc();
  for (size_t i = 0; i < sizeof(entries) / sizeof(entries[0]); ++i) check_entry(&entries[i]);
  check_sizes();
  /* with no device, a call that passes validation reports the runtime's error */
  jb_shape s = base_shape(0);
  reset_ptrs(K_PREFILL);
  jb_status st = c_prefill(&s, WS_OK);
  EXPECT(st == JB_ERR_HIP && strstr(jb_last_error(), "jb_prefill:"), "valid call without a device gave %s",
         jb_status_string(st));
  /* T = 0 takes no token pointers and no workspace */
  s.T = 0;
  reset_ptrs(K_PREFILL);
  P[0] = P[1] = P[2] = P[3] = P[4] = P[5] = P[12] = P[15] = NULL;
  st = c_prefill(&s, 0);
  EXPECT(st == JB_ERR_HIP, "empty prefill without token pointers gave %s", jb_status_string(st));
  if (fails) {
    fprintf(stderr, "%d of %d checks failed\n", fails, checks);
    return 1;
  }
  printf("host validation under sanitizers: %d checks passed\n", checks);
  return 0;
}
