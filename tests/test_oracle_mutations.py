"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one.  Every mutation is applied through monkeypatch, so the real
oracle is untouched once the test ends."""
import numpy as np
import pytest

import oracle as O
import oracle.dense_oracle as D
from tests import test_oracle_pins as P


def _expect_pin_failure(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_dropped_bias_caught(monkeypatch):
    real = D.dense_act_fwd

    def no_bias(X, W, b, act):
        return real(X, W, None, act)

    monkeypatch.setattr(O, "dense_act_fwd", no_bias)
    _expect_pin_failure(P.test_dense_fwd_brute_force, O.ACT_IDENTITY, (3, 5, 4))


def test_transposed_weight_caught(monkeypatch):
    def transposed(X, W, b, act):
        X = np.asarray(X, np.float64)
        W = np.asarray(W, np.float64)
        n = min(W.shape)
        Z = X[:, :n] @ W[:n, :n] + np.asarray(b, np.float64)[None, :n]
        return D.act_fwd(Z, act), Z

    monkeypatch.setattr(O, "dense_act_fwd", transposed)
    _expect_pin_failure(P.test_dense_fwd_brute_force, O.ACT_RELU, (4, 6, 3))


def test_gelu_grad_dropped_term_caught(monkeypatch):
    real = D.act_grad

    def wrong(z, act):
        if act == O.ACT_GELU_TANH:
            t = D._gelu_tanh_inner(np.asarray(z, np.float64))
            return 0.5 * (1.0 + t)  # the z (1 - t^2) term dropped
        return real(z, act)

    monkeypatch.setattr(O, "act_grad", wrong)
    _expect_pin_failure(P.test_act_grad_central_difference, O.ACT_GELU_TANH)


def test_vjp_wrong_sign_caught(monkeypatch):
    real = D.dense_act_vjp

    def wrong(dY, Z, X, W, act, need_dx=True, mask=None):
        dX, dW, db = real(dY, Z, X, W, act, need_dx, mask)
        return dX, -dW, db

    monkeypatch.setattr(O, "dense_act_vjp", wrong)
    _expect_pin_failure(P.test_vjp_central_difference, O.ACT_RELU)


def test_db_over_wrong_axis_caught(monkeypatch):
    real = D.dense_act_vjp

    def wrong(dY, Z, X, W, act, need_dx=True, mask=None):
        dX, dW, _ = real(dY, Z, X, W, act, need_dx, mask)
        G = np.asarray(dY, np.float64) * D.act_grad(Z, act)
        return dX, dW, G.sum(axis=1)[: dW.shape[0]]

    monkeypatch.setattr(O, "dense_act_vjp", wrong)
    _expect_pin_failure(P.test_vjp_db_is_column_sum_of_masked_grad, O.ACT_IDENTITY)


def test_xent_missing_batch_mean_caught(monkeypatch):
    real = D.softmax_xent_fwd_bwd

    def wrong(z, y):
        loss, dz, row = real(z, y)
        return loss, dz * len(y), row

    monkeypatch.setattr(O, "softmax_xent_fwd_bwd", wrong)
    _expect_pin_failure(P.test_xent_matches_library_routines)


def test_xent_wrong_label_index_caught(monkeypatch):
    def wrong(z, y):
        return D.softmax_xent_fwd_bwd(z, (np.asarray(y) + 1) % np.asarray(z).shape[1])

    monkeypatch.setattr(O, "softmax_xent_fwd_bwd", wrong)
    _expect_pin_failure(P.test_xent_matches_library_routines)


def test_adamw_missing_bias_correction_caught(monkeypatch):
    def wrong(w, g, m, v, lr, b1, b2, eps, wd, t):
        w = np.asarray(w, np.float64) * (1 - lr * wd)
        m = b1 * np.asarray(m, np.float64) + (1 - b1) * np.asarray(g)
        v = b2 * np.asarray(v, np.float64) + (1 - b2) * np.asarray(g) ** 2
        return w - lr * m / (np.sqrt(v) + eps), m, v

    monkeypatch.setattr(O, "adamw_step", wrong)
    _expect_pin_failure(P.test_adamw_step1_closed_form)


def test_adamw_coupled_decay_caught(monkeypatch):
    def coupled(w, g, m, v, lr, b1, b2, eps, wd, t):
        g = np.asarray(g, np.float64) + wd * np.asarray(w, np.float64)
        return D.adamw_step(w, g, m, v, lr, b1, b2, eps, 0.0, t)

    monkeypatch.setattr(O, "adamw_step", coupled)
    _expect_pin_failure(P.test_adamw_matches_torch_adamw_many_steps)


def test_mlp_missing_hidden_mask_caught(monkeypatch):
    real = D.dense_act_vjp

    def no_mask(dY, Z, X, W, act, need_dx=True, mask=None):
        return real(dY, Z, X, W, O.ACT_IDENTITY, need_dx, None)

    monkeypatch.setattr(D, "dense_act_vjp", no_mask)
    _expect_pin_failure(P.test_mlp_step_gradients_central_difference)


# ---- optimizer, loss and gradient-control variants

from tests import test_oracle_pins_train as PT  # noqa: E402


def test_adam_with_decoupled_decay_caught(monkeypatch):
    monkeypatch.setattr(O, "adam_step", D.adamw_step)
    _expect_pin_failure(PT.test_adam_matches_torch_adam_many_steps)


def test_clip_without_eps_caught(monkeypatch):
    monkeypatch.setattr(O, "clip_coef", lambda norm, mx: min(1.0, mx / norm))
    _expect_pin_failure(PT.test_global_norm_and_clip_coef_hand_values)


def test_norm_without_square_root_caught(monkeypatch):
    def sq(grads):
        return float(sum(np.sum(np.asarray(g, np.float64) ** 2) for g in grads))

    monkeypatch.setattr(O, "global_grad_norm", sq)
    _expect_pin_failure(PT.test_clip_matches_torch_clip_grad_norm)


def test_ema_swapped_weights_caught(monkeypatch):
    monkeypatch.setattr(O, "ema_update", lambda e, w, d: d * np.asarray(w) + (1 - d) * np.asarray(e))
    _expect_pin_failure(PT.test_ema_constant_parameter_closed_form)


def test_warmup_off_by_one_caught(monkeypatch):
    real = D.lr_at

    def wrong(kind, base, t, warmup=0, total=1, min_lr=0.0, step_size=1, gamma=1.0):
        if kind == O.LR_WARMUP_COSINE and t - 1 < warmup:
            return base * (t - 1) / warmup
        return real(kind, base, t, warmup, total, min_lr, step_size, gamma)

    monkeypatch.setattr(O, "lr_at", wrong)
    _expect_pin_failure(PT.test_lr_schedules_match_torch_schedulers)


def test_mse_missing_factor_two_caught(monkeypatch):
    real = D.mse_loss_fwd_bwd

    def wrong(p, t):
        loss, d = real(p, t)
        return loss, d / 2

    monkeypatch.setattr(O, "mse_loss_fwd_bwd", wrong)
    _expect_pin_failure(PT.test_mse_matches_torch_and_central_difference)


def test_scaler_early_growth_caught(monkeypatch):
    def update(self, found_inf):
        if found_inf:
            self.scale *= self.backoff_factor
            self.tracker = 0
            return
        self.tracker += 1
        if self.tracker >= self.growth_interval - 1:
            self.scale *= self.growth_factor
            self.tracker = 0

    monkeypatch.setattr(O.LossScaler, "update", update)
    _expect_pin_failure(PT.test_loss_scaler_hand_trajectory)


def test_norm_of_scaled_gradients_caught(monkeypatch):
    real = D.grad_control

    def wrong(scaled, max_norm=0.0, scale=1.0):
        found, _, mul = real(scaled, max_norm, scale)
        return found, O.global_grad_norm(scaled), mul

    monkeypatch.setattr(O, "grad_control", wrong)
    _expect_pin_failure(PT.test_grad_control_finite_check_and_multiplier)


def test_skipped_step_counting_caught(monkeypatch):
    real = D.mlp_train_step

    def wrong(state, *a, **k):
        out = real(state, *a, **k)
        if out["skipped"]:
            state.t += 1
        return out

    monkeypatch.setattr(O, "mlp_train_step", wrong)
    _expect_pin_failure(PT.test_mlp_scaler_skips_non_finite_step_and_backs_off)


def test_f16_overflow_to_inf_caught(monkeypatch):
    def no_saturation(a):
        f = np.asarray(a, np.float64).astype(np.float32)
        with np.errstate(over="ignore"):
            return f.astype(np.float16).astype(np.float64)

    monkeypatch.setattr(O, "round_f16_sat", no_saturation)
    _expect_pin_failure(P.test_round_f16_sat_hand_values)


def test_f16_truncation_caught(monkeypatch):
    def truncate(a):
        f = np.asarray(a, np.float64).astype(np.float32)
        u = f.view(np.uint32) & np.uint32(0xFFFFE000)  # chop the low 13 mantissa bits
        return np.clip(u.view(np.float32).astype(np.float64), -65504.0, 65504.0)

    monkeypatch.setattr(O, "round_f16_sat", truncate)
    _expect_pin_failure(P.test_round_f16_sat_matches_torch_cast_in_range)


def test_safe_scale_off_by_one_binade_caught(monkeypatch):
    real = D.f16_safe_scale
    monkeypatch.setattr(O, "f16_safe_scale", lambda a: 2.0 * real(a))
    _expect_pin_failure(P.test_f16_safe_scale_hand_values)


# ---- the rounding bands the parity tests widen comparisons by --------------

from oracle import rounding_bands as RB  # noqa: E402
from tests import test_oracle_bands as PB  # noqa: E402


def test_band_ten_times_too_wide_caught(monkeypatch):
    real = RB.dot_band
    monkeypatch.setattr(O, "relu_kink_band", lambda X, W, b, dX=None: 10.0 * real(X, W, b, dX))
    _expect_pin_failure(PB.test_dot_band_near_attained_by_ties)


def test_band_twice_too_wide_caught(monkeypatch):
    real = RB.dot_band
    monkeypatch.setattr(O, "relu_kink_band", lambda X, W, b, dX=None: 2.0 * real(X, W, b, dX))
    _expect_pin_failure(PB.test_dot_band_near_attained_by_ties)


def test_band_without_operand_deviation_caught(monkeypatch):
    real = RB.dot_band
    monkeypatch.setattr(O, "dot_band", lambda X, W, b=None, dX=None: real(X, W, b, None))
    _expect_pin_failure(PB.test_dot_band_covers_perturbed_operand)


def test_band_deviation_counted_twice_caught(monkeypatch):
    real = RB.dot_band

    def doubled(X, W, b=None, dX=None):
        extra = 0.0 if dX is None else np.asarray(dX) @ np.abs(np.asarray(W, np.float64)).T
        return real(X, W, b, dX) + extra

    monkeypatch.setattr(O, "dot_band", doubled)
    _expect_pin_failure(PB.test_dot_band_perturbation_term_is_tight)


def test_sum_band_gamma_of_fewer_terms_caught(monkeypatch):
    def short(G, h, dG=None, dh=None):
        aG = np.abs(np.asarray(G, np.float64))
        return RB.gamma(aG.shape[0] // 4) * (aG.T @ np.abs(np.asarray(h, np.float64)))

    monkeypatch.setattr(O, "sum_band", short)
    _expect_pin_failure(PB.test_sum_band_holds_and_is_near_attained)


def test_xent_band_without_logit_deviation_caught(monkeypatch):
    real = RB.xent_grad_band
    monkeypatch.setattr(O, "xent_grad_band",
                        lambda z, tau, B, scale=1.0, labels=None, form="softmax":
                        real(z, 0.0 * np.asarray(tau), B, scale, labels, form))
    _expect_pin_failure(PB.test_xent_grad_band_holds)


def test_xent_band_far_too_wide_caught(monkeypatch):
    real = RB.xent_grad_band
    monkeypatch.setattr(O, "xent_grad_band",
                        lambda z, tau, B, scale=1.0, labels=None, form="softmax":
                        10.0 * real(z, tau, B, scale, labels, form))
    _expect_pin_failure(PB.test_xent_grad_band_is_tight_for_a_dominant_class)


def test_lse_band_without_lse_deviation_caught(monkeypatch):
    """The lse form with the deviation of lse itself left out (tau only)."""
    real = RB.xent_grad_band

    def no_lambda(z, tau, B, scale=1.0, labels=None, form="softmax"):
        if form != "lse":
            return real(z, tau, B, scale, labels, form)
        z = np.asarray(z, np.float64)
        lse = O.softmax_lse(z)[:, None]
        p = np.exp(z - lse)
        dp = p * (np.exp(np.asarray(tau)) - 1.0)
        return (abs(scale) / B) * (dp + RB.gamma(4) * (1.0 + dp))

    monkeypatch.setattr(O, "xent_grad_band", no_lambda)
    _expect_pin_failure(PB.test_xent_grad_band_lse_form_is_tight)


def test_xent_band_nan_row_escaping_the_cap_caught(monkeypatch):
    """A row whose sum bound overflows (0 times inf: NaN) left out of the cap,
    as an `eps_s >= 1` test alone would leave it."""
    real = RB.xent_grad_band

    def uncapped(z, tau, B, scale=1.0, labels=None, form="softmax"):
        band = real(z, tau, B, scale, labels, form)
        t = np.asarray(tau, np.float64)
        with np.errstate(over="ignore"):
            over = ~np.isfinite(np.exp(t + t.max(axis=1, keepdims=True))).all(axis=1)
        band[over] = np.nan
        return band

    monkeypatch.setattr(O, "xent_grad_band", uncapped)
    _expect_pin_failure(PB.test_xent_grad_band_caps_rows_whose_bound_overflows)
