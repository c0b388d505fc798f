/*
 * A C11 client of libgsz that runs one synchronous ZeRO-1/2 step for every
 * owner with nothing but the C ABI of include/gsz.h and the HIP runtime: plan,
 * plan tables in its own device buffer, bucket pack of every rank's
 * per-tensor gradients, ring-order reduce-mean with the fused norm partials,
 * clip coefficient, AdamW on each owner's shard with the bf16 parameters in
 * all-gather layout.  Test infrastructure: tests/test_gpu_c_client.py writes
 * the inputs, runs this program and compares what it writes with the oracle.
 *
 * Usage: c_step_client <dir>.  <dir>/params.txt holds
 *   n_tensors world_size bucket_cap_bytes lr beta1 beta2 eps weight_decay step max_norm
 *   numel[0] ... numel[n_tensors-1]
 * and <dir>/grads_<q>.bin rank q's gradients (bf16 bits, tensors in forward
 * order, back to back), <dir>/{master,m,v}_<r>.bin owner r's shard of the
 * fp32 state.  Written: <dir>/out_g_<r>.bin, out_{master,m,v}_<r>.bin,
 * out_gathered.bin, out_partials.bin, out_clip.bin (coef, norm as floats,
 * then total as a double).  Exit status 0 on success; a failing call prints
 * its status and gsz_last_error() and exits with 2.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gsz.h"

#define MAX_T 4096
#define MAX_P 64

static void die(const char* what, int rc) {
    fprintf(stderr, "%s failed: %d (%s): %s\n", what, rc, gsz_status_string(rc), gsz_last_error());
    exit(2);
}
static void hip_check(const char* what, hipError_t e) {
    if (e != hipSuccess) {
        fprintf(stderr, "%s failed: %s\n", what, hipGetErrorString(e));
        exit(2);
    }
}
#define GSZ(call) do { int rc_ = (call); if (rc_ != GSZ_OK) die(#call, rc_); } while (0)
#define HIP(call) hip_check(#call, (call))

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
    void* buf = malloc(bytes ? bytes : 1);
    if (!buf || fread(buf, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
    fclose(f);
    return buf;
}

static void write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(buf, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
    fclose(f);
}

/* device copy of n bytes from a host buffer */
static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    HIP(hipMalloc(&d, bytes ? bytes : 16));
    if (bytes) HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static void from_device(void* host, const void* dev, size_t bytes) {
    if (bytes) HIP(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
}

int main(int argc, char** argv) {
    if (argc != 2) { fprintf(stderr, "usage: %s <dir>\n", argv[0]); return 1; }
    const char* dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/params.txt", dir);
    FILE* pf = fopen(path, "r");
    if (!pf) { fprintf(stderr, "cannot open %s\n", path); return 2; }
    int n_tensors = 0, P = 0;
    long long cap = 0, step = 0;
    double lr, b1, b2, eps, wd, max_norm;
    if (fscanf(pf, "%d %d %lld %lf %lf %lf %lf %lf %lld %lf", &n_tensors, &P, &cap, &lr, &b1, &b2,
               &eps, &wd, &step, &max_norm) != 10 || n_tensors < 0 || n_tensors > MAX_T || P < 1 ||
        P > MAX_P) {
        fprintf(stderr, "bad params.txt\n");
        return 2;
    }
    static int64_t numel[MAX_T];
    for (int t = 0; t < n_tensors; ++t) {
        long long n;
        if (fscanf(pf, "%lld", &n) != 1 || n < 0) { fprintf(stderr, "bad numel\n"); return 2; }
        numel[t] = n;
    }
    fclose(pf);

    gsz_plan* plan = NULL;
    GSZ(gsz_plan_create(numel, n_tensors, cap, P, 64, &plan));
    gsz_plan_info info;
    GSZ(gsz_plan_get_info(plan, &info));
    const int64_t S = info.shard_len, L = info.flat_len;

    hipStream_t stream;
    HIP(hipStreamCreate(&stream));
    size_t tab_bytes = 0;
    GSZ(gsz_plan_device_bytes(plan, &tab_bytes));
    void* tables = NULL;
    HIP(hipMalloc(&tables, tab_bytes));
    GSZ(gsz_plan_upload(plan, tables, tab_bytes, stream));

    /* every rank's per-tensor gradients, packed into its bucket-major buffer */
    uint16_t* flats[MAX_P];
    for (int q = 0; q < P; ++q) {
        char name[64];
        snprintf(name, sizeof name, "grads_%d.bin", q);
        uint16_t* host = read_file(dir, name, (size_t)info.n_params * 2);
        static const uint16_t* grads[MAX_T];
        static void* owned[MAX_T];
        int64_t off = 0;
        for (int t = 0; t < n_tensors; ++t) {
            owned[t] = to_device(host + off, (size_t)numel[t] * 2);
            grads[t] = owned[t];
            off += numel[t];
        }
        HIP(hipMalloc((void**)&flats[q], (size_t)L * 2 + 16));
        GSZ(gsz_bucket_pack(plan, grads, flats[q], stream));
        HIP(hipStreamSynchronize(stream));
        for (int t = 0; t < n_tensors; ++t) HIP(hipFree(owned[t]));
        free(host);
    }

    /* reduce-mean with the fused norm partial, every owner */
    size_t ws_bytes = 0;
    GSZ(gsz_workspace_bytes(S, &ws_bytes));
    void* ws = NULL;
    HIP(hipMalloc(&ws, ws_bytes));
    double* partials = NULL;
    HIP(hipMalloc((void**)&partials, (size_t)P * sizeof(double)));
    float* g[MAX_P];
    const uint16_t* contrib[MAX_P];
    for (int q = 0; q < P; ++q) contrib[q] = flats[q];
    for (int r = 0; r < P; ++r) {
        HIP(hipMalloc((void**)&g[r], (size_t)S * 4 + 16));
        GSZ(gsz_shard_reduce_mean(plan, r, contrib, GSZ_LAYOUT_BUCKET_FLAT, g[r], partials + r, ws,
                                  ws_bytes, stream));
    }

    /* clip coefficient on the device */
    float* clip = NULL;            /* coef, norm */
    double* total = NULL;
    HIP(hipMalloc((void**)&clip, 2 * sizeof(float)));
    HIP(hipMalloc((void**)&total, sizeof(double)));
    GSZ(gsz_clip_coef(partials, P, (float)max_norm, clip, clip + 1, total, stream));

    /* AdamW on every owner's shard, bf16 parameters in all-gather layout */
    gsz_adamw_hp hp = {lr, b1, b2, eps, wd, (int64_t)step};
    uint16_t* gathered = NULL;
    HIP(hipMalloc((void**)&gathered, (size_t)L * 2 + 16));
    HIP(hipMemset(gathered, 0xff, (size_t)L * 2));
    float* state[MAX_P][3];
    const char* kinds[3] = {"master", "m", "v"};
    for (int r = 0; r < P; ++r) {
        for (int k = 0; k < 3; ++k) {
            char name[64];
            snprintf(name, sizeof name, "%s_%d.bin", kinds[k], r);
            float* host = read_file(dir, name, (size_t)S * 4);
            state[r][k] = to_device(host, (size_t)S * 4);
            free(host);
        }
        GSZ(gsz_shard_adamw_step(plan, r, state[r][0], state[r][1], state[r][2], g[r], clip, &hp,
                                 gathered, NULL, stream));
    }
    HIP(hipStreamSynchronize(stream));

    /* results */
    void* buf = malloc((size_t)(L > S ? L : S) * 4 + 64);
    if (!buf) return 2;
    for (int r = 0; r < P; ++r) {
        char name[64];
        from_device(buf, g[r], (size_t)S * 4);
        snprintf(name, sizeof name, "out_g_%d.bin", r);
        write_file(dir, name, buf, (size_t)S * 4);
        for (int k = 0; k < 3; ++k) {
            from_device(buf, state[r][k], (size_t)S * 4);
            snprintf(name, sizeof name, "out_%s_%d.bin", kinds[k], r);
            write_file(dir, name, buf, (size_t)S * 4);
        }
    }
    from_device(buf, gathered, (size_t)L * 2);
    write_file(dir, "out_gathered.bin", buf, (size_t)L * 2);
    from_device(buf, partials, (size_t)P * sizeof(double));
    write_file(dir, "out_partials.bin", buf, (size_t)P * sizeof(double));
    unsigned char cl[2 * sizeof(float) + sizeof(double)];
    from_device(cl, clip, 2 * sizeof(float));
    from_device(cl + 2 * sizeof(float), total, sizeof(double));
    write_file(dir, "out_clip.bin", cl, sizeof cl);
    free(buf);

    for (int r = 0; r < P; ++r) {
        HIP(hipFree(g[r]));
        for (int k = 0; k < 3; ++k) HIP(hipFree(state[r][k]));
    }
    for (int q = 0; q < P; ++q) HIP(hipFree(flats[q]));
    HIP(hipFree(gathered));
    HIP(hipFree(clip));
    HIP(hipFree(total));
    HIP(hipFree(partials));
    HIP(hipFree(ws));
    HIP(hipFree(tables));
    HIP(hipStreamDestroy(stream));
    GSZ(gsz_plan_destroy(plan));
    printf("ok %d owners, S=%lld\n", P, (long long)S);
    return 0;
}
