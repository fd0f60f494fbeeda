/* Host-sanitizer driver of the C ABI (include/liger_attn.h): every exported call
 * with invalid, overflowing, overlapping and valid arguments. Device pointers
 * are fake (distinct 16-byte aligned addresses); the kernels are replaced by
 * launchers that report "no device", so a valid call ends in LIGER_E_HIP and
 * nothing is dereferenced. Exit status 0 when every status is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "liger_attn.h"

static int failures = 0, checks = 0;

#define P(x) ((void*)(uintptr_t)(x))
#define G ((uintptr_t)1 << 32)
#define BASE ((uintptr_t)0x100000)

static void expect(const char* what, liger_status got, liger_status want) {
    ++checks;
    const char* msg = liger_last_error();
    if (got != want) {
        ++failures;
        fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, msg);
    }
    if (want != LIGER_OK && (msg == NULL || msg[0] == '\0')) {
        ++failures;
        fprintf(stderr, "FAIL %s: no error message\n", what);
    }
}

static liger_shape shape(int64_t B, int64_t T, int32_t Hq, int32_t Hkv, int32_t d, int32_t dt) {
    liger_shape s;
    s.B = B; s.T = T; s.H_q = Hq; s.H_kv = Hkv; s.d = d; s.dtype = dt;
    return s;
}

int main(void) {
    const liger_shape ok8b = shape(1, 8192, 32, 8, 128, LIGER_BF16);
    const size_t ws = liger_attn_prefill_workspace_size(&ok8b);
    ++checks;
    if (ws == 0 || ws % 16) { ++failures; fprintf(stderr, "FAIL workspace size %zu\n", ws); }

    /* prefill: valid call reaches the launcher */
    expect("prefill valid", liger_attn_prefill(P(BASE), P(BASE + G), P(BASE + 2 * G), 0, 64, 0.5f, &ok8b,
                                               P(BASE + 3 * G), P(BASE + 4 * G), P(BASE + 5 * G), ws, NULL),
           LIGER_E_HIP);
    /* prefill: invalid arguments */
    liger_shape bad = ok8b; bad.d = 96;
    expect("prefill d=96", liger_attn_prefill(P(BASE), P(BASE + G), P(BASE + 2 * G), 0, 64, 0.5f, &bad,
                                              P(BASE + 3 * G), P(BASE + 4 * G), P(BASE + 5 * G), ws, NULL),
           LIGER_E_UNSUPPORTED);
    expect("prefill NULL shape", liger_attn_prefill(P(BASE), P(BASE), P(BASE), 0, 64, 0.5f, NULL, P(BASE + G),
                                                    P(BASE + 2 * G), NULL, 0, NULL), LIGER_E_INVALID_ARG);
    expect("prefill alias", liger_attn_prefill(P(BASE), P(BASE + G), P(BASE + 2 * G), 0, 64, 0.5f, &ok8b,
                                               P(BASE + 4096), P(BASE + 4 * G), P(BASE + 5 * G), ws, NULL),
           LIGER_E_INVALID_ARG);
    expect("prefill small ws", liger_attn_prefill(P(BASE), P(BASE + G), P(BASE + 2 * G), 0, 64, 0.5f, &ok8b,
                                                  P(BASE + 3 * G), P(BASE + 4 * G), P(BASE + 5 * G), ws - 16, NULL),
           LIGER_E_WORKSPACE);
    expect("prefill ws overlaps o", liger_attn_prefill(P(BASE), P(BASE + G), P(BASE + 2 * G), 0, 64, 0.5f, &ok8b,
                                                       P(BASE + 3 * G), P(BASE + 4 * G), P(BASE + 3 * G + 64), ws,
                                                       NULL),
           LIGER_E_INVALID_ARG);
    expect("prefill alpha nan", liger_attn_prefill(P(BASE), P(BASE + G), P(BASE + 2 * G), 0, 64, 0.0f / 0.0f, &ok8b,
                                                   P(BASE + 3 * G), P(BASE + 4 * G), P(BASE + 5 * G), ws, NULL),
           LIGER_E_INVALID_ARG);
    /* shapes whose byte counts overflow */
    const liger_shape huge = shape(65535, (int64_t)1 << 31, 65535, 65535, 128, LIGER_BF16);
    ++checks;
    if (liger_attn_prefill_backward_workspace_size(&huge) != 0) { ++failures; fprintf(stderr, "FAIL huge bwd ws\n"); }
    expect("prefill huge", liger_attn_prefill(P(BASE), P(BASE + G), P(BASE + 2 * G), 0, 64, 0.5f, &huge,
                                              P(BASE + 3 * G), P(BASE + 4 * G), P(BASE + 5 * G), SIZE_MAX, NULL),
           LIGER_E_INVALID_ARG);
    expect("backward huge", liger_attn_prefill_backward(P(BASE), P(BASE + G), P(BASE + 2 * G), P(BASE + 3 * G), 0, 64,
                                                        0.5f, &huge, P(BASE + 4 * G), P(BASE + 5 * G),
                                                        P(BASE + 6 * G), P(BASE + 7 * G), SIZE_MAX, NULL),
           LIGER_E_INVALID_ARG);
    expect("full huge", liger_attn_full_causal(P(BASE), P(BASE + G), P(BASE + 2 * G), &huge, P(BASE + 3 * G), NULL),
           LIGER_E_INVALID_ARG);

    /* stages, ex, sinks */
    expect("stages mask 0", liger_attn_prefill_stages(P(BASE), P(BASE + G), P(BASE + 2 * G), 0, 64, 0.5f, &ok8b,
                                                      P(BASE + 3 * G), P(BASE + 4 * G), P(BASE + 5 * G), ws, 0, 0,
                                                      NULL), LIGER_E_INVALID_ARG);
    expect("ex cps -1", liger_attn_prefill_ex(P(BASE), P(BASE + G), P(BASE + 2 * G), 0, 64, 0.5f, &ok8b,
                                              P(BASE + 3 * G), P(BASE + 4 * G), P(BASE + 5 * G), ws, -1, NULL),
           LIGER_E_INVALID_ARG);
    liger_sinks sk; sk.k = P(BASE + 8 * G); sk.v = P(BASE + 9 * G); sk.n = 16;
    expect("sinks valid", liger_attn_prefill_sinks(P(BASE), P(BASE + G), P(BASE + 2 * G), &sk, 1, 64, 0.5f, &ok8b,
                                                   P(BASE + 3 * G), P(BASE + 4 * G), P(BASE + 5 * G), ws, NULL),
           LIGER_E_HIP);
    sk.n = 17;
    expect("sinks n=17", liger_attn_prefill_sinks(P(BASE), P(BASE + G), P(BASE + 2 * G), &sk, 1, 64, 0.5f, &ok8b,
                                                  P(BASE + 3 * G), P(BASE + 4 * G), P(BASE + 5 * G), ws, NULL),
           LIGER_E_INVALID_ARG);

    /* decode, ring fill, continuation */
    const liger_shape dec = shape(64, 1, 32, 8, 128, LIGER_BF16);
    liger_kv_ring ring;
    ring.k = P(BASE + 10 * G); ring.v = P(BASE + 11 * G); ring.pos = (int64_t*)P(BASE + 12 * G);
    ring.sync = (uint32_t*)P(BASE + 13 * G); ring.window = 64;
    expect("decode valid", liger_attn_decode_step(P(BASE), P(BASE + G), P(BASE + 2 * G), (float*)P(BASE + 3 * G), &ring,
                                                  1, 0.5f, &dec, P(BASE + 4 * G), NULL), LIGER_E_HIP);
    ring.sync = (uint32_t*)P(BASE + 12 * G + 64 * 8 - 8);
    expect("decode pos/sync overlap", liger_attn_decode_step(P(BASE), P(BASE + G), P(BASE + 2 * G),
                                                             (float*)P(BASE + 3 * G), &ring, 1, 0.5f, &dec,
                                                             P(BASE + 4 * G), NULL), LIGER_E_INVALID_ARG);
    ring.sync = (uint32_t*)P(BASE + 13 * G);
    ring.window = 65;
    expect("decode window 65", liger_attn_decode_step(P(BASE), P(BASE + G), P(BASE + 2 * G), (float*)P(BASE + 3 * G),
                                                      &ring, 1, 0.5f, &dec, P(BASE + 4 * G), NULL),
           LIGER_E_INVALID_ARG);
    ring.window = 64;
    const liger_shape pr = shape(64, 300, 32, 8, 128, LIGER_BF16);
    expect("ring fill valid", liger_kv_ring_fill(P(BASE), P(BASE + G), &pr, &ring, NULL), LIGER_E_HIP);
    expect("ring fill k overlap", liger_kv_ring_fill(P(BASE + 10 * G + 128), P(BASE + G), &pr, &ring, NULL),
           LIGER_E_INVALID_ARG);
    const size_t wsc = liger_attn_prefill_workspace_size(&pr);
    expect("continue valid", liger_attn_prefill_continue(P(BASE), P(BASE + G), P(BASE + 2 * G), (float*)P(BASE + 3 * G),
                                                         &ring, 1, 0.5f, &pr, P(BASE + 4 * G), (float*)P(BASE + 5 * G),
                                                         P(BASE + 6 * G), wsc, NULL), LIGER_E_HIP);
    expect("continue S_T = S0", liger_attn_prefill_continue(P(BASE), P(BASE + G), P(BASE + 2 * G),
                                                             (float*)P(BASE + 3 * G), &ring, 1, 0.5f, &pr,
                                                             P(BASE + 4 * G), (float*)P(BASE + 3 * G), P(BASE + 6 * G),
                                                             wsc, NULL), LIGER_E_INVALID_ARG);

    /* full attention, backward */
    expect("full valid", liger_attn_full_causal(P(BASE), P(BASE + G), P(BASE + 2 * G), &ok8b, P(BASE + 3 * G), NULL),
           LIGER_E_HIP);
    const size_t wsb = liger_attn_prefill_backward_workspace_size(&ok8b);
    expect("backward valid", liger_attn_prefill_backward(P(BASE), P(BASE + G), P(BASE + 2 * G), P(BASE + 3 * G), 0, 64,
                                                         0.5f, &ok8b, P(BASE + 4 * G), P(BASE + 5 * G),
                                                         P(BASE + 6 * G), P(BASE + 7 * G), wsb, NULL), LIGER_E_HIP);
    liger_shape f32 = ok8b;
    f32.dtype = LIGER_F32;
    expect("backward fp32", liger_attn_prefill_backward(P(BASE), P(BASE + G), P(BASE + 2 * G), P(BASE + 3 * G), 0, 64,
                                                        0.5f, &f32, P(BASE + 4 * G), P(BASE + 5 * G), P(BASE + 6 * G),
                                                        P(BASE + 7 * G), wsb, NULL), LIGER_E_UNSUPPORTED);

    /* allocation-free prefill: limits are checked before any HIP call */
    const liger_shape big = shape(65, 64, 32, 8, 128, LIGER_BF16);
    expect("noalloc too big", liger_attn_prefill_noalloc(P(BASE), P(BASE + G), P(BASE + 2 * G), 0, 64, 0.5f, &big,
                                                         P(BASE + 3 * G), (float*)P(BASE + 4 * G), NULL),
           LIGER_E_WORKSPACE);
    ++checks;
    if (liger_attn_prefill_noalloc_max_workspace() != ((size_t)32 << 20)) { ++failures; fprintf(stderr, "FAIL max\n"); }

    printf("%d checks, %d failures\n", checks, failures);
    return failures ? 1 : 0;
}
